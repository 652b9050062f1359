// Forward attention kernels for gfx950: one fused pass per 128-row query tile
// that scans key/value blocks with the online-softmax recurrence.
//
// Method: OCANNL "Module Ir.Online_softmax", fourth rewrite bullet (the block
// fold): per key block the score tile (contraction, scale, mask), the new row
// maximum, the rescale factor, the exponentials, the rescaled sum and the
// rescaled output numerator U accumulating p * v; the last block writes
// O = U / l; a key count that is not a multiple of the block leaves a guarded
// tail whose scores are -inf.  Relations: TIGA-lang "Attention and dense
// relations" (dense, causal j <= i, varlen block-diagonal with cu_seqlens).
//
// Work decomposition (MI355X): a workgroup of 4 waves owns 128 query rows of
// one head (32 per wave).  Each wave computes the transposed score tile
// S^T = K Q^T on MFMA so that every lane owns ONE query row: the row maximum
// and row sum are in-lane reductions plus a single exchange between the two
// lane halves, and the rescale of U by alpha is a per-lane multiply.  Q lives
// in registers for the whole scan; K and V blocks are staged through LDS
// (V transposed, for the 16-bit types) with coalesced 16-byte global loads that
// are prefetched into registers one block ahead.  Workgroup index order puts
// the head index fastest, so the round-robin dispatch over the 8 XCDs keeps
// each head's K/V on one XCD's L2 when H is a multiple of 8, and causal tiles
// are issued heaviest first.
#include "attn_device.h"

namespace osattn {

constexpr int kThreads = 256;
constexpr int kBR = 128;  // query rows per workgroup

struct FwdWork {
    int h;
    int q_lo, q_hi;    // query rows [q_lo, q_hi) of this tile
    int kv_lo, kv_hi;  // keys the tile's rows may attend
    bool ok;
};

template <int MASK>
__device__ __forceinline__ FwdWork fwd_work(const FwdParams &p) {
    constexpr bool causal = MASK == kCausal || MASK == kVarlenCausal;
    constexpr bool varlen = MASK == kVarlen || MASK == kVarlenCausal;
    const int b = blockIdx.x;
    FwdWork w;
    w.h = b % p.H;
    int rest = b / p.H;
    int seq_lo = 0, seq_hi = p.n_q;
    if (varlen) {
        const Span s = seq_bounds(p.cu, rest % p.num_seqs, p.n_q);
        rest /= p.num_seqs;
        seq_lo = s.lo;
        seq_hi = s.hi;
    }
    const int tile = causal ? (p.n_tiles - 1 - rest) : rest;  // heaviest first
    w.q_lo = seq_lo + tile * kBR;
    w.q_hi = min(w.q_lo + kBR, seq_hi);
    w.ok = w.q_lo < seq_hi;
    w.kv_lo = seq_lo;
    w.kv_hi = varlen ? (causal ? w.q_hi : seq_hi) : (causal ? w.q_hi : p.n_k);
    return w;
}

// Online-softmax update of one lane's row for one key block (F4, F5): S holds
// the raw dot products of the block (masked entries -inf) and is overwritten
// with p = exp(scale * s - m_new) computed as exp2(s * c - m_new * c).
// Returns alpha, the factor that rescales the running numerator.
template <int NS>
__device__ __forceinline__ float online_update(f32x16 (&S)[NS], float &m_run, float &l_run,
                                               float c) {
    float mx = kNegInf;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[s][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));  // the other 16 keys of each group
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;  // no (-inf) - (-inf)
    const float alpha = fast_exp2((m_run - m_use) * c);
    const float mc = m_use * c;
    float rs = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pv = fast_exp2(fmaf(S[s][r], c, -mc));
            S[s][r] = pv;
            rs += pv;
        }
    l_run = l_run * alpha + rs;  // per-lane partial sum; halves merged at the end
    m_run = m_new;
    return alpha;
}

// Causal / tail mask of one block (F3).  key = k0 + 32 s + acc_row(r, g).
template <int NS, bool CAUSAL>
__device__ __forceinline__ void mask_block(f32x16 (&S)[NS], int k0, int g, int kv_hi, int qrow) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * s + acc_row(r, g);
            if (key >= kv_hi || (CAUSAL && key > qrow)) S[s][r] = kNegInf;
        }
}

// Epilogue (F7): O = U / l, m in natural-log units of the scaled score.
template <int NDT>
__device__ __forceinline__ void fwd_epilogue(const FwdParams &p, const FwdWork &w, int qrow,
                                             int g, f32x16 (&U)[NDT], float m_run,
                                             float l_run) {
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (qrow >= w.q_hi) return;
    const float inv = 1.f / l_tot;
    float *orow = p.o + (int64_t)w.h * p.o_sh + (int64_t)qrow * p.o_sn;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4 val = {U[dt][4 * j] * inv, U[dt][4 * j + 1] * inv, U[dt][4 * j + 2] * inv,
                         U[dt][4 * j + 3] * inv};
            *reinterpret_cast<f32x4 *>(orow + 32 * dt + 8 * j + 4 * g) = val;
        }
    if (g == 0) {
        p.m[(int64_t)w.h * p.n_q + qrow] = m_run * p.scale;
        p.l[(int64_t)w.h * p.n_q + qrow] = l_tot;
    }
}

// ------------------------------------------------------------ fp16 / bf16
// MFMA v_mfma_f32_32x32x16_{f16,bf16}; f32 accumulation; P rounded to T (RNE)
// as the operand of the P.V product, the row sum taken from the f32 P.
template <typename T, int D, int BC, int MASK>
__global__ void __launch_bounds__(kThreads, 2) fwd16_kernel(FwdParams p) {
    typedef typename Half8<T>::vec vec8;
    constexpr bool causal = MASK == kCausal || MASK == kVarlenCausal;
    constexpr int KCH = D / 8;                  // 16-byte chunks per K row
    constexpr int VCH = BC / 8;                 // 16-byte chunks per transposed V row
    constexpr int KLD = BC * KCH / kThreads;    // K chunks each thread stages per block
    constexpr int NS = BC / 32;                 // S^T tiles per block
    constexpr int NDT = D / 32;                 // output feature tiles
    constexpr int NKK = D / 16;                 // k-steps of K Q^T
    constexpr int NPV = BC / 16;                // k-steps of V^T P^T
    static_assert((BC / 4) * (D / 8) == kThreads, "one 4-key x 8-feature V unit per thread");
    static_assert(KLD * kThreads == BC * KCH, "K block must split evenly over the threads");

    __shared__ u32x4 sK[BC * KCH];
    __shared__ u32x4 sV[D * VCH];

    const FwdWork w = fwd_work<MASK>(p);
    if (!w.ok) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c32 = lane & 31, g = lane >> 5;
    const T *qh = static_cast<const T *>(p.q) + (int64_t)w.h * p.q_sh;
    const T *kh = static_cast<const T *>(p.k) + (int64_t)w.h * p.kv_sh;
    const T *vh = static_cast<const T *>(p.v) + (int64_t)w.h * p.kv_sh;

    // F0: this lane's query row, as the B operand (8 features per k-step).
    const int qrow = w.q_lo + wave * 32 + c32;
    const bool qok = qrow < w.q_hi;
    vec8 qreg[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
        qreg[kk] = __builtin_bit_cast(vec8, load16(qh + (int64_t)qrow * p.q_sn + 16 * kk + 8 * g, qok));

    // F1: K rows copied as 16-byte chunks; V as 4-key x 8-feature units that
    // are transposed in registers into the (feature, key-slot) LDS tile.
    const int v_d8 = tid % (D / 8), v_k4 = tid / (D / 8);
    u32x4 kreg[KLD], vreg[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int id = tid + i * kThreads, row = id / KCH, ch = id % KCH;
            const int key = k0 + row;
            kreg[i] = load16(kh + (int64_t)key * p.kv_sn + ch * 8, key < w.kv_hi);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = k0 + 4 * v_k4 + i;
            vreg[i] = load16(vh + (int64_t)key * p.kv_sn + v_d8 * 8, key < w.kv_hi);
        }
    };
    auto lds_store = [&]() {
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int id = tid + i * kThreads, row = id / KCH, ch = id % KCH;
            sK[row * KCH + swz(row, ch)] = kreg[i];
        }
        const int slot0 = key_slot(4 * v_k4);  // 4 consecutive keys -> 4 consecutive slots
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
            const unsigned a0 = vreg[0][w2], a1 = vreg[1][w2], a2 = vreg[2][w2], a3 = vreg[3][w2];
            const int d0 = v_d8 * 8 + 2 * w2, d1 = d0 + 1;
            uint2 lo, hi;
            lo.x = (a0 & 0xffffu) | (a1 << 16);
            lo.y = (a2 & 0xffffu) | (a3 << 16);
            hi.x = (a0 >> 16) | (a1 & 0xffff0000u);
            hi.y = (a2 >> 16) | (a3 & 0xffff0000u);
            reinterpret_cast<uint2 *>(&sV[d0 * VCH + swz_t(d0, slot0 >> 3)])[(slot0 >> 2) & 1] = lo;
            reinterpret_cast<uint2 *>(&sV[d1 * VCH + swz_t(d1, slot0 >> 3)])[(slot0 >> 2) & 1] = hi;
        }
    };

    f32x16 U[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) U[dt] = zero_vec<f32x16>();
    float m_run = kNegInf, l_run = 0.f;
    const float c = p.scale_log2;
    const int nblk = (w.kv_hi - w.kv_lo + BC - 1) / BC;

    gload(w.kv_lo);
    for (int kb = 0; kb < nblk; ++kb) {
        const int k0 = w.kv_lo + kb * BC;
        __syncthreads();
        lds_store();
        __syncthreads();
        if (kb + 1 < nblk) gload(k0 + BC);

        // F2: S^T = K Q^T (raw dot products).
        f32x16 S[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            S[s] = zero_vec<f32x16>();
            const u32x4 *krow = &sK[(32 * s + c32) * KCH];
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                S[s] = Half8<T>::mma(__builtin_bit_cast(vec8, krow[swz(c32, 2 * kk + g)]), qreg[kk], S[s]);
        }
        // F3: mask only blocks that straddle the diagonal or the tail.
        if (k0 + BC > w.kv_hi || (causal && k0 + BC - 1 > w.q_lo))
            mask_block<NS, causal>(S, k0, g, w.kv_hi, qrow);
        // F4, F5
        const float alpha = online_update<NS>(S, m_run, l_run, c);
        vec8 P[NPV];
#pragma unroll
        for (int t = 0; t < NPV; ++t) {
            f32x8 x;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = S[t >> 1][8 * (t & 1) + e];
            P[t] = __builtin_convertvector(x, vec8);
        }
        // F6: U = alpha U + V^T P^T.
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) U[dt] *= alpha;
#pragma unroll
        for (int t = 0; t < NPV; ++t)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const int d = 32 * dt + c32;
                const vec8 a = __builtin_bit_cast(vec8, sV[d * VCH + swz_t(d, 2 * t + g)]);
                U[dt] = Half8<T>::mma(a, P[t], U[dt]);
            }
    }
    fwd_epilogue<NDT>(p, w, qrow, g, U, m_run, l_run);
}

// ---------------------------------------------------------------------- f32
// MFMA v_mfma_f32_32x32x2_f32.  The contraction slots of K Q^T are assigned so
// that lane half g covers features [g D/2, (g+1) D/2): Q stays in registers and
// K is read in 16-byte vectors.  P stays f32.
template <int D, int BC, int MASK>
__global__ void __launch_bounds__(kThreads, D == 64 ? 2 : 1) fwd32_kernel(FwdParams p) {
    constexpr bool causal = MASK == kCausal || MASK == kVarlenCausal;
    constexpr int KCH = D / 4;                 // 16-byte chunks per row
    constexpr int LD = BC * KCH / kThreads;    // chunks per thread per tensor
    constexpr int NS = BC / 32, NDT = D / 32, NQ = D / 2, NJ = D / 8;
    static_assert(LD * kThreads == BC * KCH, "block must split evenly over the threads");

    __shared__ u32x4 sK[BC * KCH];
    __shared__ u32x4 sV[BC * KCH];

    const FwdWork w = fwd_work<MASK>(p);
    if (!w.ok) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c32 = lane & 31, g = lane >> 5;
    const float *qh = static_cast<const float *>(p.q) + (int64_t)w.h * p.q_sh;
    const float *kh = static_cast<const float *>(p.k) + (int64_t)w.h * p.kv_sh;
    const float *vh = static_cast<const float *>(p.v) + (int64_t)w.h * p.kv_sh;

    const int qrow = w.q_lo + wave * 32 + c32;
    const bool qok = qrow < w.q_hi;
    float qreg[NQ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const f32x4 x = __builtin_bit_cast(
            f32x4, load16(qh + (int64_t)qrow * p.q_sn + (D / 2) * g + 4 * j, qok));
#pragma unroll
        for (int e = 0; e < 4; ++e) qreg[4 * j + e] = x[e];
    }

    u32x4 kreg[LD], vreg[LD];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int id = tid + i * kThreads, row = id / KCH, ch = id % KCH;
            const int key = k0 + row;
            const bool ok = key < w.kv_hi;
            kreg[i] = load16(kh + (int64_t)key * p.kv_sn + ch * 4, ok);
            vreg[i] = load16(vh + (int64_t)key * p.kv_sn + ch * 4, ok);
        }
    };
    auto lds_store = [&]() {
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int id = tid + i * kThreads, row = id / KCH, ch = id % KCH;
            sK[row * KCH + swz(row, ch)] = kreg[i];
            sV[row * KCH + swz(row, ch)] = vreg[i];
        }
    };

    f32x16 U[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) U[dt] = zero_vec<f32x16>();
    float m_run = kNegInf, l_run = 0.f;
    const float c = p.scale_log2;
    const int nblk = (w.kv_hi - w.kv_lo + BC - 1) / BC;
    const float *sVf = reinterpret_cast<const float *>(sV);

    gload(w.kv_lo);
    for (int kb = 0; kb < nblk; ++kb) {
        const int k0 = w.kv_lo + kb * BC;
        __syncthreads();
        lds_store();
        __syncthreads();
        if (kb + 1 < nblk) gload(k0 + BC);

        f32x16 S[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            S[s] = zero_vec<f32x16>();
            const u32x4 *krow = &sK[(32 * s + c32) * KCH];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const f32x4 a = __builtin_bit_cast(f32x4, krow[swz(c32, (D / 8) * g + j)]);
#pragma unroll
                for (int e = 0; e < 4; ++e) S[s] = mma_f32(a[e], qreg[4 * j + e], S[s]);
            }
        }
        if (k0 + BC > w.kv_hi || (causal && k0 + BC - 1 > w.q_lo))
            mask_block<NS, causal>(S, k0, g, w.kv_hi, qrow);
        const float alpha = online_update<NS>(S, m_run, l_run, c);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) U[dt] *= alpha;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kl = 32 * s + acc_row(r, g);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const int d = 32 * dt + c32;
                    const float a = sVf[(kl * KCH + swz(kl, d >> 2)) * 4 + (d & 3)];
                    U[dt] = mma_f32(a, S[s][r], U[dt]);
                }
            }
    }
    fwd_epilogue<NDT>(p, w, qrow, g, U, m_run, l_run);
}

// ------------------------------------------------------------------ launch
template <int MASK>
static void launch_fwd_mask(int dtype, int d, const FwdParams &p, int grid, hipStream_t st) {
    const dim3 gr(grid), bl(kThreads);
    if (dtype == 1) {
        if (d == 64) hipLaunchKernelGGL((fwd16_kernel<_Float16, 64, 128, MASK>), gr, bl, 0, st, p);
        else hipLaunchKernelGGL((fwd16_kernel<_Float16, 128, 64, MASK>), gr, bl, 0, st, p);
    } else if (dtype == 2) {
        if (d == 64) hipLaunchKernelGGL((fwd16_kernel<__bf16, 64, 128, MASK>), gr, bl, 0, st, p);
        else hipLaunchKernelGGL((fwd16_kernel<__bf16, 128, 64, MASK>), gr, bl, 0, st, p);
    } else {
        if (d == 64) hipLaunchKernelGGL((fwd32_kernel<64, 64, MASK>), gr, bl, 0, st, p);
        else hipLaunchKernelGGL((fwd32_kernel<128, 32, MASK>), gr, bl, 0, st, p);
    }
}

// Host entry used by the C ABI (arguments already validated).
hipError_t launch_forward(int dtype, int d, int mask, FwdParams p, int max_seqlen,
                          hipStream_t st) {
    const int rows = (mask >= kVarlen) ? max_seqlen : p.n_q;
    p.n_tiles = (rows + kBR - 1) / kBR;
    const int64_t grid = (int64_t)p.n_tiles * p.H * (mask >= kVarlen ? p.num_seqs : 1);
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    switch (mask) {
        case kDense: launch_fwd_mask<kDense>(dtype, d, p, (int)grid, st); break;
        case kCausal: launch_fwd_mask<kCausal>(dtype, d, p, (int)grid, st); break;
        case kVarlen: launch_fwd_mask<kVarlen>(dtype, d, p, (int)grid, st); break;
        default: launch_fwd_mask<kVarlenCausal>(dtype, d, p, (int)grid, st); break;
    }
    return hipGetLastError();
}

}  // namespace osattn
