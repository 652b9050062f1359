// Forward attention kernels for gfx950: one fused pass per query tile that
// scans key/value blocks with the online-softmax recurrence.
//
// Method: OCANNL "Module Ir.Online_softmax", fourth rewrite bullet (the block
// fold): per key block the score tile (contraction, scale, mask), the new row
// maximum, the rescale factor, the exponentials, the rescaled sum and the
// rescaled output numerator U accumulating p * v; the last block writes
// O = U / l; a key count that is not a multiple of the block leaves a guarded
// tail whose scores are -inf.  Relations: TIGA-lang "Attention and dense
// relations" (dense, causal j <= i, varlen block-diagonal with cu_seqlens).
//
// Work decomposition (MI355X).  fp16/bf16: 128-row tiles of dense and causal
// problems (and of varlen problems of long sequences) run on fwd_wide_kernel,
// 8 waves per CU, each wave software-pipelined over its key chunks (see
// there).  The tiled kernel fwd16_kernel takes the rest: a workgroup of 8 or 4
// waves owns a tile of 32 RG query rows of one head (RG row groups x 8/RG key
// groups: 64- and 32-row tiles of small grids, and 128-row varlen tiles with
// two 4-wave workgroups per CU).  Each wave computes the transposed score tile S^T = K Q^T on MFMA so
// that every lane owns ONE query row: the row maximum and row sum are in-lane
// reductions plus one exchange between the two lane halves, and the rescale of U
// is a per-lane multiply.  Q lives in registers for the whole scan; K and V
// blocks go HBM/L2 -> LDS by buffer-load DMA, two stages deep, and V reaches the
// MFMA through the transposing LDS read.  The key groups of a row merge through
// LDS at the end.  f32: 4 waves own 128 rows with the 32x32x2 f32 MFMA and
// register-staged K/V.  Workgroup index order puts the head index fastest, so the
// round-robin dispatch over the 8 XCDs keeps each head's K/V on one XCD's L2 when
// H is a multiple of 8; causal tiles are paired (T-1-i, i) for equal work, and
// varlen tiles can follow a sorted work list (see the schedule kernel).
#include <type_traits>
#include <utility>

#include "attn_device.h"

namespace osattn {

constexpr int kThreads = 256;
constexpr int kBR = 128;  // query rows per workgroup
constexpr int kWideVarlenRows = 2048;  // varlen average rows per sequence for the 8-wave kernel

struct FwdWork {
    int h;
    int q_lo, q_hi;    // query rows [q_lo, q_hi) of this tile
    int kv_lo, kv_hi;  // keys the tile's rows may attend
    bool ok;
};

template <int MASK>
__device__ __forceinline__ FwdWork fwd_work(const FwdParams &p, int tile_rows = kBR) {
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
    w.q_lo = seq_lo + tile * tile_rows;
    w.q_hi = min(w.q_lo + tile_rows, seq_hi);
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
    float *orow = static_cast<float *>(p.o) + (int64_t)w.h * p.o_sh + (int64_t)qrow * p.o_sn;
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

// Split-KV partial state of one row for the key range `split`: U and the row sum
// against the exact running maximum (raw score units), in the layout the
// combine kernel reads: (splits, H, n_q, D + 4) f32 = U then {m, m, l, 0}.
template <int NDT>
__device__ __forceinline__ void fwd_partial(const FwdParams &p, const FwdWork &w, int split,
                                            int qrow, int g, f32x16 (&U)[NDT], float m_run,
                                            float l_run) {
    constexpr int D = 32 * NDT;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (qrow >= w.q_hi) return;
    float *prow = p.part + (((int64_t)split * p.H + w.h) * p.n_q + qrow) * (D + 4);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4 val = {U[dt][4 * j], U[dt][4 * j + 1], U[dt][4 * j + 2], U[dt][4 * j + 3]};
            *reinterpret_cast<f32x4 *>(prow + 32 * dt + 8 * j + 4 * g) = val;
        }
    if (g == 0) {
        const f32x4 stv = {m_run, m_run, l_tot, 0.f};
        *reinterpret_cast<f32x4 *>(prow + D) = stv;
    }
}

// ------------------------------------------------------------ fp16 / bf16
// v_mfma_f32_32x32x16_{f16,bf16}, f32 accumulation; P is rounded to T (RNE) as
// the operand of the P.V product while the row sum takes the f32 P.
//
// A workgroup of 8 (or 4) waves owns one query tile at a time (128 rows by default):
// with RG row groups, wave w serves rows 32 (w % RG) .. +32 and key group w / RG
// of every key block, so two waves per SIMD overlap one's exponentials with the
// other's MFMAs.  The key groups keep separate running states (m, l, U) that
// are merged through LDS once per tile with the same combine rule the
// recurrence uses between blocks.
//
// K and V blocks travel HBM/L2 -> LDS by buffer_load ... lds (no staging
// registers), double-buffered with one barrier per block; the buffer range
// check zero-fills rows past the tail.  Both tiles stay row-major in LDS: K is
// read as the A operand of S^T = K Q^T with 16-byte reads, V as the A operand
// of U^T = V^T P^T with ds_read_b64_tr_b16, which gathers the 8 keys of one
// feature column per lane in hardware.  Causal work items pair tile i with tile
// T-1-i so every workgroup scans T+1 blocks, which balances the launch without
// a work queue.
//
// Rescaling is lazy: the exponent reference m_ref only moves when a row's block
// maximum exceeds it by more than kLazyLog2 (so p <= 2^kLazyLog2); the exact
// row maximum is tracked beside it and l is re-expressed against it at the end.
// In exact arithmetic this is the same recurrence with a stale but consistent
// reference; it skips the per-block rescale of U for almost every block.
constexpr int kT16 = 512;
constexpr float kLazyLog2 = 8.f;

// A workgroup has NW = 8 waves and 128 KiB of LDS (one per CU), or NW = 4
// waves and 64 KiB (two per CU, so the two waves of a SIMD come from different
// workgroups and are not held in step by one barrier).  NST pipeline stages
// share the LDS: 2 stages of BC keys, or 4 stages of half as many keys each
// (deeper prefetch).  Measured on MI355X, 4 stages gained nothing at the shapes
// here (0.98x-1.03x), so launches use 2.
template <int D, int NST, int NW = 8>
struct Fwd16Cfg {
    static constexpr int LDS = NW == 8 ? 131072 : 65536;  // bytes of all stages
    static constexpr int BC = ((D == 64) ? 256 : 128) * 2 / NST * NW / 8;  // keys per block
    static constexpr int KH = BC / 2;                 // keys per wave group
    static constexpr int ROW = D * 2;                 // bytes per K / V row in LDS
    static constexpr int CPR = ROW / 16;              // 16-byte chunks per row
    static constexpr int TILE = BC * ROW;             // bytes of one K (or V) block
    static constexpr int STAGE = 2 * TILE;            // K then V
    static constexpr int NDMA = TILE / (64 * NW * 16);  // DMA instructions per tile per thread
    static constexpr int NS = KH / 32, NKK = D / 16, NDT = D / 32;  // 32-key chunks per wave
    static constexpr int NDMA_BLOCK = 2 * NDMA;      // DMA instructions per block per thread
    static_assert(NDMA * 64 * NW * 16 == TILE, "block must split evenly over the DMA lanes");
    static_assert(NST * STAGE == LDS, "stages fill the workgroup's LDS");
};

// The end-of-tile merge is shared by all waves when there are four or more key
// groups and every wave's U fits in the stages' LDS; otherwise key group 0
// merges alone.
template <int D, int NST, int NW, int RG>
constexpr bool kSharedMerge =
    NW / RG >= 4 && 8192 + NW * (D / 8) * 64 * 16 <= NST * Fwd16Cfg<D, NST, NW>::STAGE;

// Wait until at most `blocks` blocks of this thread's DMA are still in flight.
template <int NDMA_BLOCK, int NST>
__device__ __forceinline__ void wait_dma_blocks(int blocks) {
    if (NST > 2 && blocks >= 2) wait_vmcnt<2 * NDMA_BLOCK>();
    else if (NST > 2 && blocks == 1) wait_vmcnt<NDMA_BLOCK>();
    else wait_vmcnt<0>();
}

// F7 for every 16-bit tile: merge the KG = NW / RG key groups of each row
// through LDS, then O = U / l (or the split's partial state), m and l.  Every
// wave calls it after its last block; it begins and ends with a workgroup
// barrier (the stages' LDS is reused for the merge, and then by the next tile).
template <typename T, int D, int NST, int RG, int NW, bool O16>
__device__ __forceinline__ void fwd16_finish(const FwdParams &p, char *smem, int h, int q_hi,
                                             int split, int wave, int lane, int qrow,
                                             f32x16 (&U)[D / 32], float m_ref, float m_true,
                                             float l_run, float c) {
    typedef Fwd16Cfg<D, NST, NW> C;
    constexpr int KG = NW / RG;
    const int rg = wave % RG, kg = wave / RG;
    const int g = lane >> 5;
    __syncthreads();  // every wave is done with the last stage

    // F7: merge the KG key groups of each row, then O = U / l.
    l_run = xor32_sum(l_run);
    if constexpr (kSharedMerge<D, NST, NW, RG>) {
        // Four or more key groups: every wave leaves (m_ref, m_true, l) and U
        // in LDS, then the KG waves of a row group each take an equal share of
        // the 16-byte feature slots, rescale all KG states to the largest
        // reference M, sum them in group order and store their share of O (or
        // of the partial state).
        constexpr int SL = (D / 8) / KG;  // feature slots (4 features x 64 lanes) per wave
        float *st = reinterpret_cast<float *>(smem);         // (NW waves, 3, 64) floats
        f32x4 *su = reinterpret_cast<f32x4 *>(smem + 8192);  // (NW waves, D/8, 64) float4
        st[(wave * 3 + 0) * 64 + lane] = m_ref;
        st[(wave * 3 + 1) * 64 + lane] = m_true;
        st[(wave * 3 + 2) * 64 + lane] = l_run;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 v = {U[dt][4 * j], U[dt][4 * j + 1], U[dt][4 * j + 2], U[dt][4 * j + 3]};
                su[(wave * (D / 8) + dt * 4 + j) * 64 + lane] = v;
            }
        __syncthreads();
        float M_raw = kNegInf, mt = kNegInf;
#pragma unroll
        for (int k = 0; k < KG; ++k) {
            M_raw = vmax(M_raw, st[((rg + RG * k) * 3 + 0) * 64 + lane]);
            mt = vmax(mt, st[((rg + RG * k) * 3 + 1) * 64 + lane]);
        }
        const float M = (M_raw == kNegInf) ? 0.f : M_raw;
        float a[KG];
#pragma unroll
        for (int k = 0; k < KG; ++k) a[k] = fast_exp2((st[((rg + RG * k) * 3 + 0) * 64 + lane] - M) * c);
        float l = st[(rg * 3 + 2) * 64 + lane] * a[0];
#pragma unroll
        for (int k = 1; k < KG; ++k) l += st[((rg + RG * k) * 3 + 2) * 64 + lane] * a[k];
        if (qrow < q_hi) {
            const float inv = 1.f / l;
#pragma unroll
            for (int i = 0; i < SL; ++i) {
                const int sl = kg * SL + i, dt = sl >> 2, j = sl & 3;
                const int feat = 32 * dt + 8 * j + 4 * g;
                f32x4 acc = su[(rg * (D / 8) + sl) * 64 + lane] * a[0];
#pragma unroll
                for (int k = 1; k < KG; ++k) {
                    const f32x4 u = su[((rg + RG * k) * (D / 8) + sl) * 64 + lane];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = fmaf(u[e], a[k], acc[e]);
                }
                if (split >= 0) {
                    float *prow = p.part + (((int64_t)split * p.H + h) * p.n_q + qrow) * (D + 4);
                    *reinterpret_cast<f32x4 *>(prow + feat) = acc;
                } else {
                    const int64_t off = (int64_t)h * p.o_sh + (int64_t)qrow * p.o_sn + feat;
                    const f32x4 val = acc * inv;
                    if constexpr (O16) store4_16(static_cast<T *>(p.o) + off, val);
                    else *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + off) = val;
                }
            }
            if (kg == 0 && g == 0) {
                if (split >= 0) {
                    float *prow = p.part + (((int64_t)split * p.H + h) * p.n_q + qrow) * (D + 4);
                    const f32x4 stv = {M_raw, mt, l, 0.f};
                    *reinterpret_cast<f32x4 *>(prow + D) = stv;
                } else {
                    p.m[(int64_t)h * p.n_q + qrow] = mt * p.scale;
                    p.l[(int64_t)h * p.n_q + qrow] = l * fast_exp2((M - mt) * c);
                }
            }
        }
        __syncthreads();  // the next tile's prologue reuses this LDS
        return;
    }
    if constexpr (KG == 2) {
        // Two key groups: each wave leaves its row state and the half of U its
        // partner merges in LDS, then merges and stores its own half (group 0's
        // state first, as below).
        constexpr int SL = D / 16;  // 16-byte feature slots per wave: half of D / 8
        float *st = reinterpret_cast<float *>(smem);         // (NW waves, 3, 64) floats
        f32x4 *su = reinterpret_cast<f32x4 *>(smem + 8192);  // (NW waves, SL, 64) float4
        const int wp = kg == 0 ? wave + RG : wave - RG;      // the partner wave (same rows)
        st[(wave * 3 + 0) * 64 + lane] = m_ref;
        st[(wave * 3 + 1) * 64 + lane] = m_true;
        st[(wave * 3 + 2) * 64 + lane] = l_run;
        const auto put = [&](auto kgc) {  // the partner's half of U
            constexpr int K = decltype(kgc)::value;
#pragma unroll
            for (int i = 0; i < SL; ++i) {
                const int sl = (1 - K) * SL + i, dt = sl >> 2, j = sl & 3;
                const f32x4 v = {U[dt][4 * j], U[dt][4 * j + 1], U[dt][4 * j + 2], U[dt][4 * j + 3]};
                su[(wave * SL + i) * 64 + lane] = v;
            }
        };
        if (kg == 0) put(std::integral_constant<int, 0>{});
        else put(std::integral_constant<int, 1>{});
        __syncthreads();
        const float m_p = st[(wp * 3 + 0) * 64 + lane], mt_p = st[(wp * 3 + 1) * 64 + lane];
        const float l_p = st[(wp * 3 + 2) * 64 + lane];
        const float m0 = kg == 0 ? m_ref : m_p, m1 = kg == 0 ? m_p : m_ref;
        const float M_raw = vmax(m0, m1);
        const float mt = vmax(kg == 0 ? m_true : mt_p, kg == 0 ? mt_p : m_true);
        const float M = (M_raw == kNegInf) ? 0.f : M_raw;
        const float a0 = fast_exp2((m0 - M) * c), a1 = fast_exp2((m1 - M) * c);
        float l = (kg == 0 ? l_run : l_p) * a0;
        l += (kg == 0 ? l_p : l_run) * a1;
        const auto fin = [&](auto kgc) {  // this wave's half of O (or of the partial state)
            constexpr int K = decltype(kgc)::value;
            const float inv = 1.f / l;
#pragma unroll
            for (int i = 0; i < SL; ++i) {
                const int sl = K * SL + i, dt = sl >> 2, j = sl & 3;
                const int feat = 32 * dt + 8 * j + 4 * g;
                const f32x4 own = {U[dt][4 * j], U[dt][4 * j + 1], U[dt][4 * j + 2], U[dt][4 * j + 3]};
                const f32x4 par = su[(wp * SL + i) * 64 + lane];
                const f32x4 u0 = K == 0 ? own : par, u1 = K == 0 ? par : own;
                f32x4 acc = u0 * a0;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = fmaf(u1[e], a1, acc[e]);
                if (split >= 0) {
                    float *prow = p.part + (((int64_t)split * p.H + h) * p.n_q + qrow) * (D + 4);
                    *reinterpret_cast<f32x4 *>(prow + feat) = acc;
                } else {
                    const int64_t off = (int64_t)h * p.o_sh + (int64_t)qrow * p.o_sn + feat;
                    const f32x4 val = acc * inv;
                    if constexpr (O16) store4_16(static_cast<T *>(p.o) + off, val);
                    else *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + off) = val;
                }
            }
        };
        if (qrow < q_hi) {
            if (kg == 0) fin(std::integral_constant<int, 0>{});
            else fin(std::integral_constant<int, 1>{});
            if (kg == 0 && g == 0) {
                if (split >= 0) {
                    float *prow = p.part + (((int64_t)split * p.H + h) * p.n_q + qrow) * (D + 4);
                    const f32x4 stv = {M_raw, mt, l, 0.f};
                    *reinterpret_cast<f32x4 *>(prow + D) = stv;
                } else {
                    p.m[(int64_t)h * p.n_q + qrow] = mt * p.scale;
                    p.l[(int64_t)h * p.n_q + qrow] = l * fast_exp2((M - mt) * c);
                }
            }
        }
        __syncthreads();  // the next tile's prologue reuses this LDS
        return;
    }
    // One key group, or more than two without room for the shared merge:
    // groups 1..KG-1 leave (m_ref, m_true, l) and U in LDS; group 0 rescales
    // all KG states to the largest reference M and sums them in a fixed order.
    float *st = reinterpret_cast<float *>(smem);           // (NW waves, 3, 64) floats
    f32x4 *su = reinterpret_cast<f32x4 *>(smem + 8192);    // (NW - RG waves, D/8, 64) float4
    if (kg != 0) {
        st[(wave * 3 + 0) * 64 + lane] = m_ref;
        st[(wave * 3 + 1) * 64 + lane] = m_true;
        st[(wave * 3 + 2) * 64 + lane] = l_run;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f32x4 v = {U[dt][4 * j], U[dt][4 * j + 1], U[dt][4 * j + 2], U[dt][4 * j + 3]};
                su[((wave - RG) * (D / 8) + dt * 4 + j) * 64 + lane] = v;
            }
    }
    __syncthreads();
    if (kg == 0) {
        float M_raw = m_ref, mt = m_true;
#pragma unroll
        for (int k = 1; k < KG; ++k) {
            M_raw = vmax(M_raw, st[((rg + RG * k) * 3 + 0) * 64 + lane]);
            mt = vmax(mt, st[((rg + RG * k) * 3 + 1) * 64 + lane]);
        }
        const float M = (M_raw == kNegInf) ? 0.f : M_raw;
        const float a0 = fast_exp2((m_ref - M) * c);
        float l = l_run * a0;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) U[dt] *= a0;
#pragma unroll
        for (int k = 1; k < KG; ++k) {
            const int w = rg + RG * k;
            const float ak = fast_exp2((st[(w * 3 + 0) * 64 + lane] - M) * c);
            l += st[(w * 3 + 2) * 64 + lane] * ak;
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 u = su[((w - RG) * (D / 8) + dt * 4 + j) * 64 + lane];
#pragma unroll
                    for (int e = 0; e < 4; ++e) U[dt][4 * j + e] = fmaf(u[e], ak, U[dt][4 * j + e]);
                }
        }
        if (split >= 0 && qrow < q_hi) {
            // Partial state of this key range: U and l against reference M_raw.
            float *prow = p.part + (((int64_t)split * p.H + h) * p.n_q + qrow) * (D + 4);
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 val = {U[dt][4 * j], U[dt][4 * j + 1], U[dt][4 * j + 2], U[dt][4 * j + 3]};
                    *reinterpret_cast<f32x4 *>(prow + 32 * dt + 8 * j + 4 * g) = val;
                }
            if (g == 0) {
                f32x4 stv = {M_raw, mt, l, 0.f};
                *reinterpret_cast<f32x4 *>(prow + D) = stv;
            }
        } else if (qrow < q_hi) {
            const float inv = 1.f / l;
            const int64_t off = (int64_t)h * p.o_sh + (int64_t)qrow * p.o_sn;
            if constexpr (O16) {  // O in the input dtype: the same values, rounded once
                T *orow = static_cast<T *>(p.o) + off;
#pragma unroll
                for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const f32x4 val = {U[dt][4 * j] * inv, U[dt][4 * j + 1] * inv,
                                           U[dt][4 * j + 2] * inv, U[dt][4 * j + 3] * inv};
                        store4_16(orow + 32 * dt + 8 * j + 4 * g, val);
                    }
            } else {
                float *orow = static_cast<float *>(p.o) + off;
#pragma unroll
                for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const f32x4 val = {U[dt][4 * j] * inv, U[dt][4 * j + 1] * inv,
                                           U[dt][4 * j + 2] * inv, U[dt][4 * j + 3] * inv};
                        *reinterpret_cast<f32x4 *>(orow + 32 * dt + 8 * j + 4 * g) = val;
                    }
            }
            if (g == 0) {
                p.m[(int64_t)h * p.n_q + qrow] = mt * p.scale;
                p.l[(int64_t)h * p.n_q + qrow] = l * fast_exp2((M - mt) * c);
            }
        }
    }
    __syncthreads();  // the next tile's prologue reuses this LDS
}

// The NW waves of a workgroup form RG row groups of 32 query rows (a tile of
// 32 RG rows) times KG = NW / RG key groups; key group kg takes keys
// [kg KH, (kg + 1) KH) of every block, and the KG partial states of a row are
// merged through LDS at the end.  Launches use RG = 4 (128-row tiles) unless
// such tiles are too few to occupy the device.
// split < 0: write O, m, l.  split >= 0: write this key range's partial state.
// O16: O is written in T (the same f32 values rounded once) instead of f32.
template <typename T, int D, int MASK, int NST, int RG, int NW = 8,
          bool O16 = false>
__device__ __forceinline__ void fwd16_tile(const FwdParams &p, char *smem, int h, int q_lo,
                                           int q_hi, int kv_lo, int kv_hi, int split) {
    typedef Fwd16Cfg<D, NST, NW> C;
    typedef typename Half8<T>::vec vec8;
    constexpr bool causal = MASK == kCausal || MASK == kVarlenCausal;
    constexpr int KG = NW / RG, KH = C::BC / KG, NS = KH / 32;  // keys, 32-key chunks per wave
    static_assert(RG * KG == NW && NS * 32 == KH && NS >= 1, "wave layout must tile the block");
    static_assert(8192 + (NW - RG) * (D / 8) * 64 * 16 <= NST * C::STAGE, "merge buffers fit in LDS");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rg = wave % RG, kg = wave / RG;
    const int c32 = lane & 31, g = lane >> 5;
    constexpr int esz = (int)sizeof(T);

    // F0: this lane's query row as the B operand (zero past the tile end).
    const int qrow = q_lo + 32 * rg + c32;
    const T *qb = static_cast<const T *>(p.q) + (int64_t)h * p.q_sh + (int64_t)q_lo * p.q_sn;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (int64_t)(q_hi - q_lo) * p.q_sn * esz);
    vec8 qreg[C::NKK];
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk)
        qreg[kk] = __builtin_bit_cast(vec8, bload16(rq, ((32 * rg + c32) * (int)p.q_sn + 16 * kk + 8 * g) * esz));

    const T *kh = static_cast<const T *>(p.k) + (int64_t)h * p.kv_sh;
    const T *vh = static_cast<const T *>(p.v) + (int64_t)h * p.kv_sh;
    const int kv_sn = (int)p.kv_sn;

    // F1: DMA block [k0, k0 + BC) of K and V into stage `buf`.  DMA
    // instruction i of this wave fills LDS bytes [(NW i + wave) 1 KiB, +1 KiB)
    // of each tile; each lane fetches the global chunk its swizzled LDS slot
    // holds.  Rows at or past kv_hi arrive as zeros.
    int dma_off[C::NDMA];
#pragma unroll
    for (int i = 0; i < C::NDMA; ++i) {
        const int byte = (NW * i + wave) * 1024 + 16 * lane;
        const int row = byte / C::ROW, pch = (byte % C::ROW) / 16;
        (void)pch;
        dma_off[i] = row * kv_sn * esz;  // + logical chunk, per tile below
    }
    auto issue = [&](int k0, int buf) {
        const int64_t bytes = (int64_t)(kv_hi - k0) * kv_sn * esz;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kh + (int64_t)k0 * kv_sn, bytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vh + (int64_t)k0 * kv_sn, bytes);
        char *sk = smem + buf * C::STAGE;
        char *sv = sk + C::TILE;
#pragma unroll
        for (int i = 0; i < C::NDMA; ++i) {
            const int byte = (NW * i + wave) * 1024 + 16 * lane;
            const int row = byte / C::ROW, pch = (byte % C::ROW) / 16;
            dma16(rk, sk + (NW * i + wave) * 1024, dma_off[i] + swz_k<C::ROW>(row, pch) * 16);
            dma16(rv, sv + (NW * i + wave) * 1024, dma_off[i] + swz_vt<C::ROW>(row, pch) * 16);
        }
    };

    f32x16 U[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) U[dt] = zero_vec<f32x16>();
    float m_ref = kNegInf, m_true = kNegInf, l_run = 0.f;
    const float c = p.scale_log2;
    const int nblk = (kv_hi - kv_lo + C::BC - 1) / C::BC;
    const int wrow_lo = q_lo + 32 * rg, wrow_hi = wrow_lo + 31;

    // Prefetch distance NST - 1 blocks.
    for (int j = 0; j < NST - 1 && j < nblk; ++j) issue(kv_lo + j * C::BC, j);
    for (int j = 0; j < nblk; ++j) {
        // Block j has landed (this thread's DMA) and, after the barrier, for
        // every thread; every wave has also finished reading block j-1, so
        // its stage can take block j + NST - 1.
        wait_dma_blocks<C::NDMA_BLOCK, NST>(min(NST - 2, nblk - 1 - j));
        bare_barrier();
        if (j + NST - 1 < nblk) issue(kv_lo + (j + NST - 1) * C::BC, (j + NST - 1) % NST);

        const int k0 = kv_lo + j * C::BC;
        const int kw0 = k0 + kg * KH;  // first key of this wave's group
        const char *sk = smem + (j % NST) * C::STAGE;
        const char *sv = sk + C::TILE;
        if (kw0 < kv_hi && (!causal || kw0 <= wrow_hi)) {
            // The wave's KH keys are processed as 32-key chunks, software
            // pipelined: chunk cc+1's S^T MFMAs are issued before chunk cc's
            // exponentials so the two overlap in the same scheduling region.
            auto qk = [&](int cc) {  // F2: S^T = K Q^T for one 32-key chunk
                f32x16 S = zero_vec<f32x16>();
                const int row = kg * KH + 32 * cc + c32;
                const char *krow = sk + row * C::ROW;
#pragma unroll
                for (int kk = 0; kk < C::NKK; ++kk) {
                    const vec8 a = *reinterpret_cast<const vec8 *>(krow + swz_k<C::ROW>(row, 2 * kk + g) * 16);
                    S = Half8<T>::mma(a, qreg[kk], S);
                }
                return S;
            };
            f32x16 S = qk(0);
#pragma unroll
            for (int cc = 0; cc < NS; ++cc) {
                const int kc0 = kw0 + 32 * cc;
                // F3: mask chunks that cross the tail or the diagonal.
                if (kc0 + 32 > kv_hi || (causal && kc0 + 31 > wrow_lo)) {
                    f32x16 Sm[1] = {S};
                    mask_block<1, causal>(Sm, kc0, g, kv_hi, qrow);
                    S = Sm[0];
                }
                // F4: chunk row maximum (in-lane, then the other lane half).
                float t[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    t[i] = vmax(vmax(S[4 * i], S[4 * i + 1]), vmax(S[4 * i + 2], S[4 * i + 3]));
                float mx = vmax(vmax(t[0], t[1]), vmax(t[2], t[3]));
                mx = xor32_max(mx);
                m_true = vmax(m_true, mx);
                // F5 (lazy): move the exponent reference only on a large increase.
                if (__any((mx - m_ref) * c > kLazyLog2)) {
                    const float m_new = vmax(m_ref, mx);
                    const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2((m_ref - m_new) * c);
#pragma unroll
                    for (int dt = 0; dt < C::NDT; ++dt) U[dt] *= alpha;
                    l_run *= alpha;
                    m_ref = m_new;
                }
                const float mc = (m_ref == kNegInf) ? 0.f : m_ref * c;
                f32x16 Sn;
                if (cc + 1 < NS) Sn = qk(cc + 1);
                float ps[4];
                vec8 P[2];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    f32x8 x;
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = fast_exp2(fmaf(S[8 * hf + e], c, -mc));
                    ps[2 * hf] = (x[0] + x[1]) + (x[2] + x[3]);
                    ps[2 * hf + 1] = (x[4] + x[5]) + (x[6] + x[7]);
                    P[hf] = __builtin_convertvector(x, vec8);
                }
                l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
                // F6: U += V^T P^T over the chunk's two 16-key slices; slice hf
                // holds keys 32 cc + 16 hf + 8 x + 4 g + 0..3 (x = 0, 1).
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int r0 = kg * KH + 32 * cc + 16 * hf + 4 * g + ((lane & 15) >> 2);
                    const int cq = lane & 3, hh = (lane >> 4) & 1;
#pragma unroll
                    for (int dt = 0; dt < C::NDT; ++dt) {
                        const int ch = 4 * dt + 2 * hh + (cq >> 1);
                        const i16x4 lo = lds_read_tr16(sv + r0 * C::ROW + swz_vt<C::ROW>(r0, ch) * 16 + 8 * (cq & 1));
                        const i16x4 hi = lds_read_tr16(sv + (r0 + 8) * C::ROW + swz_vt<C::ROW>(r0 + 8, ch) * 16 + 8 * (cq & 1));
                        const vec8 a = __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                        U[dt] = Half8<T>::mma(a, P[hf], U[dt]);
                    }
                }
                if (cc + 1 < NS) S = Sn;
            }
        }
    }
    fwd16_finish<T, D, NST, RG, NW, O16>(p, smem, h, q_hi, split, wave, lane, qrow, U, m_ref,
                                         m_true, l_run, c);
}

// Split-KV combine: one pass over a row's partial states (U_s, l_s against
// reference m_s) with the rule the recurrence uses between blocks -- a running
// reference M, rescale by 2^((M_old - M) c) when it grows, add U_s 2^((m_s - M) c)
// -- then O = U / l, m = the largest exact row maximum, l re-expressed against
// it.  A workgroup of 256 threads covers 256 / (D / 4) rows, one float4 of each
// row per thread, and loads the splits eight at a time: decode-like shapes
// have few rows and many splits, and the split loop's memory latency was their
// bound (8 x 128 queries x 16384 keys, D = 128, 32 splits: forward 43.0 ->
// 27.1 us against 8 threads per row and 4 loads in flight; 16 at a time spill).
template <int D> constexpr int kCombineTPR = D / 4;                   // threads per row
template <int D> constexpr int kCombineRows = 256 / kCombineTPR<D>;  // rows per workgroup
constexpr int kCombineBatch = 8;  // splits whose loads are in flight together

// OT: the type of O (f32, or the 16-bit input type).
template <int D, typename OT>
__global__ void __launch_bounds__(256) fwd_combine_kernel(FwdParams p) {
    constexpr int QD = D / kCombineTPR<D>;  // features per thread
    static_assert(QD % 4 == 0, "whole float4 per thread");
    const int h = blockIdx.x % p.H, grp = blockIdx.x / p.H;
    const int row = grp * kCombineRows<D> + threadIdx.x / kCombineTPR<D>, part = threadIdx.x % kCombineTPR<D>;
    if (row >= p.n_q) return;
    const float c = p.scale_log2;
    const int64_t split_stride = (int64_t)p.H * p.n_q * (D + 4);
    const float *base = p.part + ((int64_t)h * p.n_q + row) * (D + 4);
    float acc[QD];
#pragma unroll
    for (int d = 0; d < QD; ++d) acc[d] = 0.f;
    float M = kNegInf, MT = kNegInf, L = 0.f;
    // Splits in groups of kCombineBatch: all of a group's loads are issued
    // before the first is used (a split index past the end re-reads the last
    // split and is skipped), so the serial chain is one memory latency per group.
    for (int s0 = 0; s0 < p.splits; s0 += kCombineBatch) {
        f32x4 stv[kCombineBatch], u[kCombineBatch][QD / 4];
#pragma unroll
        for (int k = 0; k < kCombineBatch; ++k) {
            const float *ps = base + min(s0 + k, p.splits - 1) * split_stride;
            stv[k] = *reinterpret_cast<const f32x4 *>(ps + D);
#pragma unroll
            for (int i = 0; i < QD / 4; ++i) u[k][i] = *reinterpret_cast<const f32x4 *>(ps + part * QD + 4 * i);
        }
#pragma unroll
        for (int k = 0; k < kCombineBatch; ++k) {
            if (s0 + k >= p.splits) break;
            MT = fmaxf(MT, stv[k][1]);
            const float Mn = fmaxf(M, stv[k][0]);
            if (Mn == kNegInf) continue;  // nothing admitted so far
            const float a_old = fast_exp2((M - Mn) * c), a_new = fast_exp2((stv[k][0] - Mn) * c);
            L = L * a_old + stv[k][2] * a_new;
#pragma unroll
            for (int i = 0; i < QD / 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[4 * i + e] = acc[4 * i + e] * a_old + u[k][i][e] * a_new;
            M = Mn;
        }
    }
    const float inv = 1.f / L;
    OT *orow = static_cast<OT *>(p.o) + (int64_t)h * p.o_sh + (int64_t)row * p.o_sn + part * QD;
#pragma unroll
    for (int i = 0; i < QD / 4; ++i) {
        f32x4 v = {acc[4 * i] * inv, acc[4 * i + 1] * inv, acc[4 * i + 2] * inv, acc[4 * i + 3] * inv};
        if constexpr (sizeof(OT) == 4) *reinterpret_cast<f32x4 *>(orow + 4 * i) = v;
        else store4_16(orow + 4 * i, v);
    }
    if (part == 0) {
        p.m[(int64_t)h * p.n_q + row] = MT * p.scale;
        p.l[(int64_t)h * p.n_q + row] = L * fast_exp2((M - MT) * c);
    }
}

// ------------------------------------------------------- varlen work list
// The hardware deals a grid's workgroups out in index order, and each XCD deals
// its share to its shader engines in turn, waiting for the next engine in line
// to have room.  On the natural varlen grid (head, sequence, tile pair) the
// same sequences keep landing on the same engine, so one engine can hold most
// of the long items while the others idle.  This kernel writes the varlen
// items -- tile pairs (T-1-i, i) of one sequence, as in the causal grid -- as a
// list ordered by the number of key blocks the pair scans, largest first: the
// largest items start first and consecutive workgroups carry similar work.
// Each entry holds the sequence bounds and both tiles, so a workgroup needs one
// 16-byte load to start.  One workgroup builds the list with a counting sort in
// LDS.  The order among items of equal size depends on LDS atomics; that
// changes which workgroup computes a tile, never the tile's result.
constexpr int kSchedThreads = 1024;

// Key blocks that query tile t of a length-len sequence scans.
template <int BC, bool CAUSAL>
__device__ __forceinline__ int tile_blocks(int t, int len) {
    return t < 0 ? 0 : ((CAUSAL ? min((t + 1) * kBR, len) : len) + BC - 1) / BC;
}

template <int BC, bool CAUSAL>
__global__ void __launch_bounds__(kSchedThreads) varlen_schedule_kernel(FwdParams p) {
    constexpr int PER = kSchedBins / kSchedThreads;
    static_assert(PER * kSchedThreads == kSchedBins, "bins must split evenly over the threads");
    __shared__ int cnt[kSchedBins];
    __shared__ int wtot[kSchedThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    for (int i = tid; i < kSchedBins; i += kSchedThreads) cnt[i] = 0;
    __syncthreads();
    const auto bin = [&](int s_lo, int len, int i, int T) {
        const int t0 = T - 1 - i, t1 = (i == t0) ? -1 : i;
        const int w = tile_blocks<BC, CAUSAL>(t0, len) + tile_blocks<BC, CAUSAL>(t1, len);
        return min(w >> p.sched_shift, kSchedBins - 1);
    };
    for (int s = tid; s < p.num_seqs; s += kSchedThreads) {
        const Span sq = seq_bounds(p.cu, s, p.n_q);
        const int len = sq.hi - sq.lo, T = (len + kBR - 1) / kBR;
        for (int i = 0; i < (T + 1) / 2; ++i) atomicAdd(&cnt[bin(sq.lo, len, i, T)], 1);
    }
    __syncthreads();
    // Exclusive scan from the top bin down: cnt[b] becomes bin b's first slot.
    int v[PER], run = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        v[i] = cnt[kSchedBins - 1 - (tid * PER + i)];
        run += v[i];
    }
    int incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) wtot[wv] = incl;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kSchedThreads / 64; ++w) {
        const int t = wtot[w];
        base += (w < wv) ? t : 0;
        total += t;
    }
    int ex = base + incl - run;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        cnt[kSchedBins - 1 - (tid * PER + i)] = ex;
        ex += v[i];
    }
    const int count = min(total, p.sched_max);
    if (tid == 0) p.sched[0] = count;
    __syncthreads();
    // Place the items; slots past sched_max (reachable only with malformed
    // cu_seqlens) are dropped, and unused slots get an empty entry.
    int4 *items = reinterpret_cast<int4 *>(p.sched + 4);
    for (int s = tid; s < p.num_seqs; s += kSchedThreads) {
        const Span sq = seq_bounds(p.cu, s, p.n_q);
        const int len = sq.hi - sq.lo, T = (len + kBR - 1) / kBR;
        for (int i = 0; i < (T + 1) / 2; ++i) {
            const int pos = atomicAdd(&cnt[bin(sq.lo, len, i, T)], 1);
            const int t0 = T - 1 - i;
            if (pos < p.sched_max) items[pos] = make_int4(sq.lo, sq.hi, t0, i == t0 ? -1 : i);
        }
    }
    for (int i = count + tid; i < p.sched_max; i += kSchedThreads) items[i] = make_int4(0, 0, -1, -1);
}

// A varlen work item: sequence rows [lo, hi) and its tiles t0, t1 (t1 < 0:
// one tile; t0 < 0: no work) of kBR rows.
struct VarlenItem {
    int lo, hi, t0, t1;
};

// Varlen item `rest` of one head: from the sorted work list (p.sched), from a
// ranking done here (p.sched_inline: up to 64 sequences), or from the natural
// (sequence, pair) grid.  Uniform across the workgroup: the result is taken
// into scalar registers.
__device__ __forceinline__ VarlenItem varlen_item_lanes(const FwdParams &p, int rest);
__device__ __forceinline__ VarlenItem varlen_item(const FwdParams &p, int rest) {
    const VarlenItem it = varlen_item_lanes(p, rest);
    return {__builtin_amdgcn_readfirstlane(it.lo), __builtin_amdgcn_readfirstlane(it.hi),
            __builtin_amdgcn_readfirstlane(it.t0), __builtin_amdgcn_readfirstlane(it.t1)};
}
__device__ __forceinline__ VarlenItem varlen_item_lanes(const FwdParams &p, int rest) {
    if (p.sched_inline) {
        // Item `rest` in a list of the tile pairs (T-1-i, i) that takes the
        // sequences by tile count, most first (ties: lower index first), and
        // each sequence's pairs in order of i; a pair scans about T + 1 key
        // blocks, so this is the sorted work list without a separate launch.
        // Lane s < num_seqs (at most 64) holds sequence s; every wave computes
        // the same answer.
        const int lane = threadIdx.x & 63, S = p.num_seqs;
        int lo = 0, hi = 0;
        if (lane < S) {
            const Span sp = seq_bounds(p.cu, lane, p.n_q);
            lo = sp.lo;
            hi = sp.hi;
        }
        const int nt = (hi - lo + kBR - 1) / kBR, npair = (nt + 1) / 2;
        const int key = (nt << 6) | (63 - lane);  // distinct per lane; nt < 2^24
        int before = 0;                          // pairs listed ahead of this sequence's
        for (int s2 = 0; s2 < S; ++s2) {
            const int ks = __shfl(key, s2), ns = __shfl(npair, s2);
            before += ks > key ? ns : 0;
        }
        const uint64_t own = __ballot(lane < S && rest >= before && rest < before + npair);
        if (own == 0) return {0, 0, -1, -1};  // past the last item
        const int src = __ffsll((unsigned long long)own) - 1;
        const int s_nt = __shfl(nt, src), i = rest - __shfl(before, src);
        const int ta = s_nt - 1 - i;
        return {__shfl(lo, src), __shfl(hi, src), ta, (i == ta) ? -1 : i};
    }
    if (p.sched) {  // item `rest` of the sorted work list
        const int4 it = reinterpret_cast<const int4 *>(p.sched + 4)[rest];
        return {it.x, it.y, it.z, it.w};
    }
    // pair (T-1-i, i) of sequence rest % num_seqs; the grid walks i downwards
    // from the middle tiles of the longest sequence
    const Span sq = seq_bounds(p.cu, rest % p.num_seqs, p.n_q);
    const int ntile = (sq.hi - sq.lo + kBR - 1) / kBR;
    const int i = (p.n_tiles + 1) / 2 - 1 - rest / p.num_seqs;
    if (i >= (ntile + 1) / 2) return {0, 0, -1, -1};
    const int t0 = ntile - 1 - i;
    return {sq.lo, sq.hi, t0, (i == t0) ? -1 : i};
}

// NW = 4: two workgroups per CU, so each wave may use at most 256 registers.
template <typename T, int D, int MASK, int NST, int RG, int NW = 8, bool O16 = false>
__global__ void __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) fwd16_kernel(FwdParams p) {
    constexpr bool causal = MASK == kCausal || MASK == kVarlenCausal;
    constexpr bool varlen = MASK == kVarlen || MASK == kVarlenCausal;
    constexpr int TR = 32 * RG;  // query rows per tile
    static_assert(!varlen || TR == kBR, "varlen tiles are kBR rows");
    __shared__ __attribute__((aligned(16))) char smem[NST * Fwd16Cfg<D, NST, NW>::STAGE];
    const int b = blockIdx.x;
    if (!causal && !varlen && p.splits > 1) {
        // Split-KV item; the split index varies slowest so that all splits of
        // a tile land on one XCD when H * n_tiles is a multiple of 8.
        const int items = p.H * p.n_tiles;
        const int split = b / items, r = b % items;
        const int h = r % p.H, tile = r / p.H;
        const int q_lo = tile * TR, q_hi = min(q_lo + TR, p.n_q);
        const int k_lo = split * p.split_len, k_hi = min(k_lo + p.split_len, p.n_k);
        fwd16_tile<T, D, MASK, NST, RG, NW, O16>(p, smem, h, q_lo, q_hi, k_lo, k_hi, split);
        return;
    }
    const int h = b % p.H;
    int rest = b / p.H;
    if constexpr (varlen) {
        const VarlenItem it = varlen_item(p, rest);
#pragma unroll 1
        for (int k = 0; k < 2; ++k) {
            const int tile = k == 0 ? it.t0 : it.t1;
            if (tile < 0) break;
            const int q_lo = it.lo + tile * TR, q_hi = min(q_lo + TR, it.hi);
            if (q_lo >= q_hi) break;
            fwd16_tile<T, D, MASK, NST, RG, NW, O16>(p, smem, h, q_lo, q_hi, it.lo, causal ? q_hi : it.hi, -1);
        }
        return;
    }
    int t0, t1;
    if (causal && !p.pair) {
        // one tile per workgroup, heaviest (last) tiles first: for grids too
        // small to fill the device, where a pair would double the serial work
        t0 = p.n_tiles - 1 - rest;
        t1 = -1;
    } else if (causal) {
        // pair (T-1-i, i): equal work per causal pair
        const int i = rest;
        if (i >= (p.n_tiles + 1) / 2) return;
        t0 = p.n_tiles - 1 - i;
        t1 = (i == t0) ? -1 : i;
    } else {
        t0 = rest;
        t1 = -1;
    }
#pragma unroll 1
    for (int k = 0; k < 2; ++k) {
        const int tile = k == 0 ? t0 : t1;
        if (tile < 0) break;
        const int q_lo = tile * TR, q_hi = min(q_lo + TR, p.n_q);
        fwd16_tile<T, D, MASK, NST, RG, NW, O16>(p, smem, h, q_lo, q_hi, 0, causal ? q_hi : p.n_k, -1);
    }
}

// The varlen work list on its own (the fp16/bf16 backward orders its tile pairs
// with it): the same kernel and key block as the forward of width d.
// Key block of the 16-bit forward for width d and NW waves per workgroup.
// ------------------------------------------------ pipelined waves at D = 128
// The 128-row tile at D = 128 (dense and causal relations), run by 8 waves,
// two per SIMD: wave w serves rows 32 (w % 4) .. +32 of the tile and key group
// w / 4, i.e. keys [64 kg, 64 kg + 64) of every 128-key block, as two 32-key
// chunks.
//
// Each wave runs a software pipeline over its chunks s = 0, 1, ...: step s
// computes the softmax of chunk s on the vector ALU while the same wave's
// MFMAs compute the next chunk's scores S(s+1) and add the previous chunk's
// P(s-1) V to U.  The three are independent, so the exponentials issue beside
// the MFMAs, and every operand is read from LDS four reads ahead of its use.
// A wave overlaps its own vector ALU work with its MFMAs, but one wave issues
// that work at about one instruction per 5 clocks (measured: 16 MFMAs with 8
// FMAs each take 43 clocks per MFMA in one wave, 32 alone); the second wave of
// the SIMD fills the issue gaps (two such waves: both MFMA streams at full
// rate).  The waves of a SIMD that split the phases instead -- one all MFMA,
// the other all vector ALU -- do not overlap at all (77 clocks per pair).
//
// K and V blocks use separate two-slot rings.  K(b) is read by the score
// MFMAs of steps 2b-1 and 2b, V(b) by the P.V MFMAs of steps 2b+1 and 2b+2.
// At the start of each odd step 2b-1 a wave waits for its own copies of K(b)
// and V(b-1), meets the others at a barrier, and starts K(b+1) into K(b-1)'s
// slot and V(b) into V(b-2)'s, one copy instruction per MFMA slot: every wave
// last read both in step 2b-2, and both copies have two steps to land.  One barrier per block.  The copies are
// inline assembly: the compiler, which would make any LDS read wait for every
// LDS copy in flight, then leaves their ordering to the explicit waits and
// barriers.
//
// Exponent reference.  The recurrence rescales U whenever a row maximum grows;
// here each row's reference is the maximum of its first chunk and never moves,
// so U is never rescaled and the loop carries no branch that writes it.  The
// exponentials 2^((s - m_ref) c) <= 2^((m_true - m_ref) c) are exact up to
// rounding like those of any reference at or below the true maximum, and safe
// from overflow while (m_true - m_ref) c stays below a bound B: the P operand
// is at most 2^B, and U and l stay below 2^B n max|v|.  B = 64 for bf16 (whose
// exponent range is f32's) and 15 for fp16 (largest finite value 65504, just
// under 2^16).  Every chunk checks that bound; if any row of the tile exceeds
// it (scores that grow by 10 or more natural-log units along the keys), the
// workgroup recomputes the tile with each row's exact maximum as its reference,
// found first by a pass of score MFMAs alone.  The two key groups of a row
// merge through LDS at the end.
//
// The steps below are written for RH 32-row halves per wave, RH = 1.  With
// RH = 2 (4 waves, one per SIMD, 64 rows each) every K or V operand read feeds
// two MFMAs, half the LDS bytes per MFMA, but the one wave per SIMD issues all
// of the vector ALU work: 3-5 % slower (causal N=4096 H=16 bf16 77.0 against
// 73.9 us).
template <int D_>
struct WideCfg {
    static constexpr int D = D_, BC = 128, ROW = 2 * D, KH = 64, RH = 1;
    static constexpr int NW = 8 / RH, RGN = NW / 2;   // waves; row groups (x 2 key groups)
    static constexpr int NKK = D / 16, NDT = D / 32;  // 16-feature slices, 32-feature tiles
    static constexpr int RPK = 1024 / ROW, CPR = ROW / 16;  // rows per KiB, 16-byte chunks per row
    static constexpr int NSL = RH * (NKK + 2 * NDT);  // MFMA slots of a pipeline step
    static constexpr int KT = BC * ROW;  // bytes of one K (or V) block
    static constexpr int KS0 = 0, KS1 = KT, VS0 = 2 * KT, VS1 = 3 * KT;  // LDS slots
    static constexpr int NDMA = KT / (64 * NW * 16);  // 16-byte copies per lane per block
    static constexpr int STATS = 4 * KT;                // merge statistics, 8 KiB
    static constexpr int FLAG = STATS + 8192;           // recompute flag
    static constexpr int LDS = FLAG + 16;
    // largest (m_true - m_ref) c kept on this path, by input type
    template <typename T> static constexpr float kRefLog2 = std::is_same<T, _Float16>::value ? 15.f : 64.f;
};

// Returns false when the tile must be recomputed (see above); then nothing
// of o, m, l (or the partial state) has been written by this call.  With
// exact_ref the reference of each row is its exact maximum, and the call
// always succeeds.  q_lo - kv_lo is a multiple of 128 and, for the causal
// relations, kv_hi = q_hi, so only the last block can cross the diagonal or
// the tail.
// The key groups' merge of a tile whose waves own 32 rows each (8 waves):
// wave (rg, kg) finalizes the feature tiles kg NH .. kg NH + NH - 1 (NH = NDT / 2)
// of its rows.  It hands its other tiles, and per row m_ref, m_true and l, to
// its partner (rg, 1 - kg) through region (rg, 1 - kg) of the merge buffer
// (NH 4 KiB each) and takes the partner's from region (rg, kg), which it then
// reuses to turn its O tiles into whole-row stores.  Returns false (nothing
// written) when a wave raised the recompute flag.
template <typename T, int D, bool O16>
__device__ __forceinline__ bool wide_merge_rows32(const FwdParams &p, char *mbuf, char *stats,
                                                  int *flag, int h, int q_hi, int split,
                                                  int wrow_lo, int rg, int kg, int lane,
                                                  f32x16 (&U)[D / 32], float m_ref, float m_true,
                                                  float l_tot, float c) {
    constexpr int NH = D / 64;         // feature tiles each wave finalizes
    constexpr int RW = NH * 4 * 64;    // float4 per region
    constexpr int CH = D / 8;          // 16-byte chunks per row of this wave's half of O
    const int c32 = lane & 31, g = lane >> 5;
    f32x4 *give = reinterpret_cast<f32x4 *>(mbuf) + (rg * 2 + 1 - kg) * RW + lane;
    const f32x4 *take = reinterpret_cast<const f32x4 *>(mbuf) + (rg * 2 + kg) * RW + lane;
    f32x4 *sb = reinterpret_cast<f32x4 *>(stats) + lane;
    const auto hand = [&](auto d0c) {
        constexpr int d0 = decltype(d0c)::value;
#pragma unroll
        for (int t2 = 0; t2 < NH; ++t2)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 val = {U[d0 + t2][4 * j], U[d0 + t2][4 * j + 1], U[d0 + t2][4 * j + 2],
                                   U[d0 + t2][4 * j + 3]};
                give[(t2 * 4 + j) * 64] = val;
            }
    };
    if (kg == 0) hand(std::integral_constant<int, NH>{});
    else hand(std::integral_constant<int, 0>{});
    const f32x4 mine = {m_ref, m_true, l_tot, 0.f};
    sb[(rg * 2 + kg) * 64] = mine;
    wait_lgkmcnt0();
    bare_barrier();
    if (*flag) {
        bare_barrier();  // every wave has read the flag before the LDS is reused
        return false;
    }
    const f32x4 st = sb[(rg * 2 + 1 - kg) * 64];
    const float M = vmax(m_ref, st[0]);
    const float a0 = fast_exp2((m_ref - M) * c), a1 = fast_exp2((st[0] - M) * c);
    const float lt = l_tot * a0 + st[2] * a1;
    const float mt = vmax(m_true, st[1]);
    const int qrow = wrow_lo + c32;
    // Physical chunk of logical chunk ch in row r of a region (rows of CH
    // chunks): 16 lanes that write one chunk of 16 rows, or read the chunks of
    // a row (or two), hit 16 distinct bank groups.
    const auto pch = [](int r, int ch) { return CH == 16 ? (ch ^ (r & 15)) : (ch ^ ((r >> 1) & 7)); };
    const auto finish = [&](auto d0c) {
        constexpr int d0 = decltype(d0c)::value;
        if (split >= 0) {
            if (qrow >= q_hi) return;
            float *prow = p.part + (((int64_t)split * p.H + h) * p.n_q + qrow) * (D + 4);
#pragma unroll
            for (int t2 = 0; t2 < NH; ++t2)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 u1 = take[(t2 * 4 + j) * 64];
                    f32x4 val;
#pragma unroll
                    for (int e = 0; e < 4; ++e) val[e] = U[d0 + t2][4 * j + e] * a0 + u1[e] * a1;
                    *reinterpret_cast<f32x4 *>(prow + 32 * (d0 + t2) + 8 * j + 4 * g) = val;
                }
            if (kg == 0 && g == 0) {
                const f32x4 stv = {M, mt, lt, 0.f};
                *reinterpret_cast<f32x4 *>(prow + D) = stv;
            }
            return;
        }
        const float b0 = a0 / lt, b1 = a1 / lt;
        f32x4 val[NH][4];
#pragma unroll
        for (int t2 = 0; t2 < NH; ++t2)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 u1 = take[(t2 * 4 + j) * 64];
#pragma unroll
                for (int e = 0; e < 4; ++e) val[t2][j][e] = U[d0 + t2][4 * j + e] * b0 + u1[e] * b1;
            }
        if (kg == 0 && g == 0 && qrow < q_hi) {
            p.m[(int64_t)h * p.n_q + qrow] = mt * p.scale;
            p.l[(int64_t)h * p.n_q + qrow] = lt * fast_exp2((M - mt) * c);
        }
        // Row c32 of the region: CH chunks of 4 features (this wave's D / 2),
        // chunk 8 t2 + 2 j + g.
        wait_lgkmcnt0();  // every read of the region has returned
        f32x4 *obuf = reinterpret_cast<f32x4 *>(mbuf) + (rg * 2 + kg) * RW;
#pragma unroll
        for (int t2 = 0; t2 < NH; ++t2)
#pragma unroll
            for (int j = 0; j < 4; ++j) obuf[c32 * CH + pch(c32, 8 * t2 + 2 * j + g)] = val[t2][j];
        wait_lgkmcnt0();
        if constexpr (O16) {
            constexpr int LPR = CH / 2, RPI = 64 / LPR;  // lanes per row, rows per instruction
#pragma unroll
            for (int i = 0; i < 32 / RPI; ++i) {  // 8 values per lane
                const int r = RPI * i + lane / LPR, c8 = lane % LPR;
                const f32x4 lo = obuf[r * CH + pch(r, 2 * c8)];
                const f32x4 hi = obuf[r * CH + pch(r, 2 * c8 + 1)];
                if (wrow_lo + r < q_hi) {
                    T *dst = static_cast<T *>(p.o) + (int64_t)h * p.o_sh + (int64_t)(wrow_lo + r) * p.o_sn +
                             (D / 2) * kg + 8 * c8;
                    store4_16(dst, lo);
                    store4_16(dst + 4, hi);
                }
            }
        } else {
            constexpr int RPI = 64 / CH;  // rows per instruction
#pragma unroll
            for (int i = 0; i < 32 / RPI; ++i) {  // 4 values per lane
                const int r = RPI * i + lane / CH, ch = lane % CH;
                const f32x4 v4 = obuf[r * CH + pch(r, ch)];
                if (wrow_lo + r < q_hi)
                    *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + (int64_t)h * p.o_sh +
                                               (int64_t)(wrow_lo + r) * p.o_sn + (D / 2) * kg + 4 * ch) = v4;
            }
        }
    };
    if (kg == 0) finish(std::integral_constant<int, 0>{});
    else finish(std::integral_constant<int, NH>{});
    // The next tile's copies reuse the slots: a barrier without a memory
    // fence (the stores above need not have landed; every LDS read here has).
    wait_lgkmcnt0();
    bare_barrier();
    return true;
}

template <typename T, int D, int MASK, bool O16>
__device__ __forceinline__ bool fwd_wide_tile(const FwdParams &p, char *smem, int h, int q_lo,
                                              int q_hi, int kv_lo, int kv_hi, int split,
                                              bool exact_ref) {
    typedef WideCfg<D> C;
    constexpr int RH = C::RH, ROW = C::ROW;
    typedef typename Half8<T>::vec vec8;
    constexpr bool causal = MASK == kCausal || MASK == kVarlenCausal;
    constexpr int NDT = C::NDT, NKK = C::NKK, esz = (int)sizeof(T);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg = wave % C::RGN, kg = wave / C::RGN;  // row group of 32 RH rows, key group
    const int c32 = lane & 31, g = lane >> 5;
    const float c = p.scale_log2;
    const int nblk = (kv_hi - kv_lo + C::BC - 1) / C::BC;
    const int wrow_lo = q_lo + 32 * RH * rg;

    const T *kh = static_cast<const T *>(p.k) + (int64_t)h * p.kv_sh;
    const T *vh = static_cast<const T *>(p.v) + (int64_t)h * p.kv_sh;
    const int rowb = (int)p.kv_sn * esz;  // bytes between key rows (at most 4 MiB)
    const uint32_t lds0 = (uint32_t)(uintptr_t)(OSATTN_LDS char *)smem;

    // F1: copy i of this wave fills bytes [(NW i + wave) KiB, +1 KiB) of a
    // block, i.e. rows RPK (NW i + wave) + L / CPR, 16-byte chunk L % CPR of
    // each (stored at its swizzled place, the same for every copy i); rows at
    // or past kv_hi arrive as zeros.
    const int drow = C::RPK * wave + lane / C::CPR;
    const int k_goff = drow * rowb + swz_k<ROW>(drow, lane % C::CPR) * 16;
    const int v_goff = drow * rowb + swz_vt<ROW>(drow, lane % C::CPR) * 16;
    const int max_rows = 0x7ffffff0 / rowb;  // rows one buffer resource may span
    const auto desc = [&](const T *base, int b) {  // block b of K or V
        const int k0 = kv_lo + b * C::BC;
        return rsrc_words(base + (int64_t)k0 * p.kv_sn, min(kv_hi - k0, max_rows) * rowb);
    };
    const auto copy_one = [&](const i32x4 &r, uint32_t slot, int goff, int i) {
        dma16_asm(r, lds0 + slot + (C::NW * i + wave) * 1024, goff + C::RPK * C::NW * i * rowb);
    };
    const auto copy = [&](const T *base, int b, uint32_t slot, int goff) {
        asm volatile("" : "+v"(goff));  // per-copy offsets are formed here, not hoisted
        const i32x4 r = desc(base, b);
#pragma unroll
        for (int i = 0; i < C::NDMA; ++i) copy_one(r, slot, goff, i);
    };

    // F0: this lane's query rows (one per half) as B operands (zero past the
    // tile end).
    copy(kh, 0, C::KS0, k_goff);
    const T *qb = static_cast<const T *>(p.q) + (int64_t)h * p.q_sh + (int64_t)q_lo * p.q_sn;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (int64_t)(q_hi - q_lo) * p.q_sn * esz);
    vec8 qreg[RH][NKK];
#pragma unroll
    for (int qh = 0; qh < RH; ++qh)
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            qreg[qh][kk] = __builtin_bit_cast(
                vec8, bload16(rq, ((32 * RH * rg + 32 * qh + c32) * (int)p.q_sn + 16 * kk + 8 * g) * esz));
    if (tid == 0) *reinterpret_cast<int *>(smem + C::FLAG) = 0;  // read after the merge barrier
    wait_vmcnt<0>();  // Q and K(0)
    float m_init[RH];
#pragma unroll
    for (int qh = 0; qh < RH; ++qh) m_init[qh] = kNegInf;
    if (exact_ref) {
        // F2-F4 alone: each row's exact maximum over its admitted keys, from
        // the same MFMA products (K read straight from memory in the A
        // operand layout) as the pass below computes.
        for (int k0 = kv_lo; k0 < kv_hi; k0 += 32) {
            if (causal && k0 > wrow_lo + 32 * RH - 1) break;
            const __amdgpu_buffer_rsrc_t rk =
                make_rsrc(kh + (int64_t)k0 * p.kv_sn, (int64_t)(kv_hi - k0) * rowb);
            f32x16 S[RH];
#pragma unroll
            for (int qh = 0; qh < RH; ++qh) S[qh] = zero_vec<f32x16>();
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const vec8 a = __builtin_bit_cast(vec8, bload16(rk, c32 * rowb + (16 * kk + 8 * g) * esz));
#pragma unroll
                for (int qh = 0; qh < RH; ++qh) S[qh] = Half8<T>::mma(a, qreg[qh][kk], S[qh]);
            }
#pragma unroll
            for (int qh = 0; qh < RH; ++qh) {
                f32x16 Sm[1] = {S[qh]};
                mask_block<1, causal>(Sm, k0, g, kv_hi, wrow_lo + 32 * qh + c32);
                float mx = kNegInf;
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = vmax(mx, Sm[0][r]);
                m_init[qh] = vmax(m_init[qh], xor32_max(mx));
            }
        }
    }
    if (nblk > 1) copy(kh, 1, C::KS1, k_goff);
    copy(vh, 0, C::VS0, v_goff);

    // LDS operand addresses.  K row KH kg + 32 cc + c32 of a slot, 16-byte
    // chunk 2 kk + g, swizzled with (row & 15) = (c32 & 15): the same place for
    // both cc.  V: rows r0 = KH kg + 32 cc + 16 hf + 4 g + (L % 16) / 4 and
    // r0 + 8, feature chunk 4 dt + 2 ((L / 16) & 1) + (L & 3) / 2, swizzled
    // with (r0 & 3) = (L / 4) & 3.  ka and va hold slot 0 of their ring (the
    // driver flips the slot bit); cc, hf and the +8 rows are immediate offsets.
    int ka[NKK], va[NDT];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) ka[kk] = (C::KH * kg + c32) * ROW + swz_k<ROW>(c32, 2 * kk + g) * 16;
    {
        const int vr = C::KH * kg + 4 * g + ((lane & 15) >> 2);
        const int cq = lane & 3, hh = (lane >> 4) & 1;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            va[dt] = C::VS0 + vr * ROW + swz_vt<ROW>(vr, 4 * dt + 2 * hh + (cq >> 1)) * 16 + 8 * (cq & 1);
    }
    const auto kread = [&](int kk, int off) {
        return *reinterpret_cast<const vec8 *>(smem + ka[kk] + off);
    };
    const auto vread = [&](int dt, int off) {
        const i16x4 lo = lds_read_tr16(smem + va[dt] + off);
        const i16x4 hi = lds_read_tr16(smem + va[dt] + off + 8 * ROW);
        return __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    f32x16 U[RH][NDT];
#pragma unroll
    for (int qh = 0; qh < RH; ++qh)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) U[qh][dt] = zero_vec<f32x16>();
    float m_ref[RH], m_true[RH], l_run[RH], mc[RH], thr[RH];
#pragma unroll
    for (int qh = 0; qh < RH; ++qh) {
        m_ref[qh] = 0.f;
        m_true[qh] = kNegInf;
        l_run[qh] = 0.f;
        mc[qh] = 0.f;
        thr[qh] = 0.f;
    }
    bool bail = false;
    f32x16 SA[RH], SB[RH];
    vec8 PA[RH][2], PB[RH][2];

    bare_barrier();  // every wave's part of K(0) has landed
#pragma unroll
    for (int qh = 0; qh < RH; ++qh) SA[qh] = zero_vec<f32x16>();
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        const vec8 a = kread(kk, 0);
#pragma unroll
        for (int qh = 0; qh < RH; ++qh) SA[qh] = Half8<T>::mma(a, qreg[qh][kk], SA[qh]);
    }

    // One pipeline step; its parity fixes the buffers and the 32-key chunk of
    // the reads at compile time, the slots come from ka and va.  Flags: HS,
    // S(s+1) exists; HP, P(s-1) exists; MK, chunk s may need masking (only
    // the last block's chunks can); CK / CV, the block boundary starts
    // K((s+3)/2) / V((s+1)/2); FIRST, step 0 sets the reference.
    // (Sc, Pc): chunk s's scores and probabilities; Sn receives S(s+1); Pp
    // holds P(s-1).  Even steps use (SA, PA), odd ones (SB, PB).
    const auto step_body = [&](auto ODDc, auto HSc, auto HPc, auto MKc, auto CKc, auto CVc,
                               auto FIRSTc, int s, f32x16 (&Sc)[RH], f32x16 (&Sn)[RH],
                               vec8 (&Pc)[RH][2], vec8 (&Pp)[RH][2]) {
        constexpr bool ODD = decltype(ODDc)::value, HS = decltype(HSc)::value;
        constexpr bool HP = decltype(HPc)::value, MK = decltype(MKc)::value;
        constexpr bool CK = decltype(CKc)::value, CV = decltype(CVc)::value;
        constexpr bool FIRST = decltype(FIRSTc)::value;
        // S(s+1) and P(s-1) V read chunk 0 of their block on odd steps, 1 on even.
        constexpr int KOFF = ODD ? 0 : 32 * ROW;
        constexpr int VOFF = ODD ? 0 : 32 * ROW;
        // Block boundary (odd steps): K((s+1)/2) and V((s-1)/2) have landed;
        // the copies of K((s+3)/2) and V((s+1)/2) are issued one per slot in
        // slots 0 .. 15, beside the MFMAs.
        i32x4 rk = {0, 0, 0, 0}, rv = {0, 0, 0, 0};
        uint32_t ksl = 0, vsl = 0;
        int kgo = k_goff, vgo = v_goff;
        if constexpr (ODD) {
            const int b = (s + 1) >> 1;
            wait_vmcnt<0>();
            bare_barrier();
            if constexpr (CK) {
                rk = desc(kh, b + 1);
                ksl = ((b + 1) & 1) ? C::KS1 : C::KS0;
                asm volatile("" : "+v"(kgo));  // per-copy offsets are formed here, not hoisted
            }
            if constexpr (CV) {
                rv = desc(vh, b);
                vsl = (b & 1) ? C::VS1 : C::VS0;
                asm volatile("" : "+v"(vgo));
            }
        }
        if constexpr (MK) {  // F3: chunks that cross the tail or the diagonal
            const int kc0 = kv_lo + (s >> 1) * C::BC + C::KH * kg + 32 * (s & 1);
#pragma unroll
            for (int qh = 0; qh < RH; ++qh) {
                const int r_lo = wrow_lo + 32 * qh;
                if (kc0 + 32 > kv_hi || (causal && kc0 + 31 > r_lo)) {
                    f32x16 Sm[1] = {Sc[qh]};
                    mask_block<1, causal>(Sm, kc0, g, kv_hi, r_lo + c32);
                    Sc[qh] = Sm[0];
                }
            }
        }
        // The step's MFMAs in issue order: operand read j feeds MFMAs RH j ..
        // RH j + RH - 1 (one per row half).  The reads for S(s+1) come first (K, 16
        // features kk per read), so that S(s+1) is complete long before the
        // next step reads it, then those for P(s-1) V (V, 32 features dt,
        // 16-key half hf).  Slot i issues read i / RH + FD; every slot then
        // issues its MFMA and its share of the softmax; a scheduling fence
        // after each slot keeps that order (it bounds the operands in flight).
        constexpr int NRD = (HS ? NKK : 0) + (HP ? 2 * NDT : 0);  // operand reads
        constexpr int FD = 4;                             // reads in flight ahead of use
        // read code: kk < NKK = K with kk, NKK + NDT hf + dt = V of (dt, hf)
        constexpr auto rdc = [](int j) { return HS ? j : NKK + j; };
        vec8 opnd[FD + 1];
        const auto fetch = [&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if constexpr (j < NRD) {
                constexpr int o = rdc(j);
                if constexpr (o < NKK) opnd[j % (FD + 1)] = kread(o, KOFF);
                else opnd[j % (FD + 1)] = vread((o - NKK) % NDT, VOFF + 16 * ROW * ((o - NKK) / NDT));
            }
        };
        const auto mma = [&](auto ic) {
            constexpr int i = decltype(ic)::value, j = i / RH, qh = i % RH;
            if constexpr (j < NRD) {
                constexpr int o = rdc(j);
                if constexpr (o < NKK)
                    Sn[qh] = Half8<T>::mma(opnd[j % (FD + 1)], qreg[qh][o], o == 0 ? zero_vec<f32x16>() : Sn[qh]);
                else
                    U[qh][(o - NKK) % NDT] = Half8<T>::mma(opnd[j % (FD + 1)], Pp[qh][(o - NKK) / NDT],
                                                           U[qh][(o - NKK) % NDT]);
            }
        };
        const auto dma = [&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (ODD && CK && i < C::NDMA) copy_one(rk, ksl, kgo, i);
            if constexpr (ODD && CV && i >= C::NDMA && i < 2 * C::NDMA) copy_one(rv, vsl, vgo, i - C::NDMA);
        };
        float t[RH][4], ps[RH][4], y[RH][16];
        f32x8 x[RH][2];
        // Softmax of chunk s in 16 pieces per row half, slot i taking pieces
        // PPS (i / RH) .. + PPS - 1 of row half i % RH: F4 (chunk maximum; on
        // step 0 it becomes the reference), then F5 (probabilities: f32 into
        // l, rounded to T as the P.V operand).  Each exponential is taken one
        // piece after the multiply-add that forms its argument.
        constexpr int PPS = 16 * RH / C::NSL;  // pieces per slot
        const auto piece = [&](auto qhc, auto pcc) {
            constexpr int qh = decltype(qhc)::value, pc = decltype(pcc)::value;
            const f32x16 &S = Sc[qh];
            if constexpr (pc == 0) {
                t[qh][0] = vmax(vmax(S[0], S[1]), vmax(S[2], S[3]));
                t[qh][1] = vmax(vmax(S[4], S[5]), vmax(S[6], S[7]));
            } else if constexpr (pc == 1) {
                t[qh][2] = vmax(vmax(S[8], S[9]), vmax(S[10], S[11]));
                t[qh][3] = vmax(vmax(S[12], S[13]), vmax(S[14], S[15]));
            } else if constexpr (pc == 2) {
                const float mx = xor32_max(vmax(vmax(t[qh][0], t[qh][1]), vmax(t[qh][2], t[qh][3])));
                m_true[qh] = vmax(m_true[qh], mx);
                if constexpr (FIRST) {
                    // A row with no admitted key in this chunk (a key group
                    // above the diagonal of the first tile) takes a finite
                    // stand-in: its exponentials are 0 and any later admitted
                    // key exceeds thr, which hands the tile back.
                    const float base = exact_ref ? m_init[qh] : mx;
                    m_ref[qh] = base == kNegInf ? -1e30f : base;
                    mc[qh] = m_ref[qh] * c;
                    thr[qh] = exact_ref ? __builtin_inff() : m_ref[qh] + C::template kRefLog2<T> / c;
                } else {
                    bail |= mx > thr[qh];
                }
            } else if constexpr (pc >= 3 && pc <= 11) {
                if constexpr (pc >= 4) {
                    constexpr int e0 = 2 * (pc - 4);
                    x[qh][e0 >> 3][e0 & 7] = fast_exp2(y[qh][e0]);
                    x[qh][e0 >> 3][(e0 & 7) + 1] = fast_exp2(y[qh][e0 + 1]);
                }
                if constexpr (pc <= 10) {
                    constexpr int e1 = 2 * (pc - 3);
                    y[qh][e1] = fmaf(S[e1], c, -mc[qh]);
                    y[qh][e1 + 1] = fmaf(S[e1 + 1], c, -mc[qh]);
                }
            } else if constexpr (pc == 12 || pc == 13) {
                constexpr int hf = pc - 12;
                const f32x8 &v = x[qh][hf];
                ps[qh][2 * hf] = (v[0] + v[1]) + (v[2] + v[3]);
                ps[qh][2 * hf + 1] = (v[4] + v[5]) + (v[6] + v[7]);
                Pc[qh][hf] = __builtin_convertvector(v, vec8);
            } else if constexpr (pc == 14) {
                l_run[qh] += (ps[qh][0] + ps[qh][1]) + (ps[qh][2] + ps[qh][3]);
            }
        };
        const auto valu = [&](auto ic) {
            constexpr int i = decltype(ic)::value, qh = i % RH, p0 = PPS * (i / RH);
            for_each_index([&](auto kc) { piece(std::integral_constant<int, qh>{},
                                                std::integral_constant<int, p0 + decltype(kc)::value>{}); },
                           std::make_integer_sequence<int, PPS>{});
        };
        const auto slot = [&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i % RH == 0) fetch(std::integral_constant<int, i / RH + FD>{});
            dma(ic);
            mma(ic);
            valu(ic);
            __builtin_amdgcn_sched_barrier(0);
        };
        for_each_index(fetch, std::make_integer_sequence<int, FD>{});
        for_each_index(slot, std::make_integer_sequence<int, C::NSL>{});
    };
    using Y = std::true_type;
    using N = std::false_type;
    using E = std::false_type;  // even step
    using O = std::true_type;   // odd step
    const auto step = [&](auto ODDc, auto HSc, auto HPc, auto MKc, auto CKc, auto CVc, auto FIRSTc,
                          int s) {
        if constexpr (!decltype(ODDc)::value)
            step_body(ODDc, HSc, HPc, MKc, CKc, CVc, FIRSTc, s, SA, SB, PA, PB);
        else
            step_body(ODDc, HSc, HPc, MKc, CKc, CVc, FIRSTc, s, SB, SA, PB, PA);
    };
    const auto flip_k = [&]() {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) ka[kk] ^= C::KT;
    };
    const auto flip_v = [&]() {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) va[dt] ^= C::KT;
    };
    // Steps 0 .. 2 nblk - 1, then P(2 nblk - 1) V.  Block b's scores are
    // computed by steps 2b-1 and 2b (K slot b & 1), its P.V products by steps
    // 2b+1 and 2b+2 (V slot b & 1): ka flips before each odd step from step 1
    // on, va after each even step from step 2 on.  Only the last block's
    // chunks can need a mask; its steps run outside the loop, which is then
    // free of branches.
    if (nblk == 1) step(E{}, Y{}, N{}, Y{}, N{}, N{}, Y{}, 0);
    else step(E{}, Y{}, N{}, N{}, N{}, N{}, Y{}, 0);
    int b = 1;
    if (nblk > 2) {
#pragma unroll 1
        do {
            flip_k();
            step(O{}, Y{}, Y{}, N{}, Y{}, Y{}, N{}, 2 * b - 1);
            step(E{}, Y{}, Y{}, N{}, N{}, N{}, N{}, 2 * b);
            flip_v();
        } while (++b < nblk - 1);
    }
    if (nblk > 1) {  // the last block: b = nblk - 1
        flip_k();
        step(O{}, Y{}, Y{}, N{}, N{}, Y{}, N{}, 2 * b - 1);
        step(E{}, Y{}, Y{}, Y{}, N{}, N{}, N{}, 2 * b);
        flip_v();
    }
    step(O{}, N{}, Y{}, Y{}, N{}, N{}, N{}, 2 * nblk - 1);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)  // P(2 nblk - 1) V: chunk 1 of the last block
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const vec8 a = vread(dt, 32 * ROW + 16 * ROW * hf);
#pragma unroll
            for (int qh = 0; qh < RH; ++qh) U[qh][dt] = Half8<T>::mma(a, PB[qh][hf], U[qh][dt]);
        }
    // F7: merge the two key groups of each row through LDS, into the K
    // slots: every wave finished its K reads before the last odd step's
    // barrier.  A wave that saw a row exceed the reference bound raises the
    // flag before the merge barrier, and then every wave hands the tile back.
    float l_tot[RH];
#pragma unroll
    for (int qh = 0; qh < RH; ++qh) l_tot[qh] = xor32_sum(l_run[qh]);  // the lane halves' keys
    int *flag = reinterpret_cast<int *>(smem + C::FLAG);
    if (__any(bail) && lane == 0) *flag = 1;
    return wide_merge_rows32<T, D, O16>(p, smem + C::KS0, smem + C::STATS, flag, h, q_hi, split, wrow_lo,
                                     rg, kg, lane, U[0], m_ref[0], m_true[0], l_tot[0], c);
}

// A tile the wide routine hands back is run again with exact references (one
// body of the routine in the kernel: the retry is the loop's second pass).
template <typename T, int D, int MASK, bool O16>
__device__ __forceinline__ void fwd_wide_or_retry(const FwdParams &p, char *smem, int h, int q_lo,
                                                  int q_hi, int kv_lo, int kv_hi, int split) {
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass)
        if (fwd_wide_tile<T, D, MASK, O16>(p, smem, h, q_lo, q_hi, kv_lo, kv_hi, split, pass == 1)) break;
}

// The dense and causal 16-bit forward at D = 128 with 128-row tiles: one
// workgroup of 8 waves per CU.  Work items as in fwd16_kernel: split-KV items
// (dense), causal tile pairs (T-1-i, i) or single tiles heaviest first, dense
// tiles.
template <typename T, int D, int MASK, bool O16>
__global__ void __launch_bounds__(64 * WideCfg<D>::NW, 1) fwd_wide_kernel(FwdParams p) {
    constexpr bool causal = MASK == kCausal || MASK == kVarlenCausal;
    constexpr bool varlen = MASK == kVarlen || MASK == kVarlenCausal;
    __shared__ __attribute__((aligned(16))) char smem[WideCfg<D>::LDS];
    const int b = blockIdx.x;
    if constexpr (varlen) {
        const VarlenItem it = varlen_item(p, b / p.H);
#pragma unroll 1
        for (int k = 0; k < 2; ++k) {
            const int tile = k == 0 ? it.t0 : it.t1;
            if (tile < 0) break;
            const int q_lo = it.lo + tile * kBR, q_hi = min(q_lo + kBR, it.hi);
            if (q_lo >= q_hi) break;
            fwd_wide_or_retry<T, D, MASK, O16>(p, smem, b % p.H, q_lo, q_hi, it.lo, causal ? q_hi : it.hi, -1);
        }
        return;
    }
    if (!causal && p.splits > 1) {
        const int items = p.H * p.n_tiles;
        const int split = b / items, r = b % items;
        const int h = r % p.H, tile = r / p.H;
        const int q_lo = tile * kBR, q_hi = min(q_lo + kBR, p.n_q);
        const int k_lo = split * p.split_len, k_hi = min(k_lo + p.split_len, p.n_k);
        fwd_wide_or_retry<T, D, MASK, O16>(p, smem, h, q_lo, q_hi, k_lo, k_hi, split);
        return;
    }
    const int h = b % p.H, rest = b / p.H;
    int t0, t1 = -1;
    if (causal && p.pair) {
        if (rest >= (p.n_tiles + 1) / 2) return;
        t0 = p.n_tiles - 1 - rest;
        t1 = (rest == t0) ? -1 : rest;
    } else {
        t0 = causal ? p.n_tiles - 1 - rest : rest;
    }
#pragma unroll 1
    for (int k = 0; k < 2; ++k) {
        const int tile = k == 0 ? t0 : t1;
        if (tile < 0) break;
        const int q_lo = tile * kBR, q_hi = min(q_lo + kBR, p.n_q);
        fwd_wide_or_retry<T, D, MASK, O16>(p, smem, h, q_lo, q_hi, 0, causal ? q_hi : p.n_k, -1);
    }
}

int fwd16_block_keys(int d, int waves) {
    if (d == 64) return waves == 4 ? Fwd16Cfg<64, 2, 4>::BC : Fwd16Cfg<64, 2>::BC;
    return waves == 4 ? Fwd16Cfg<128, 2, 4>::BC : Fwd16Cfg<128, 2>::BC;
}

// The schedule kernel for a key block of bc keys (64, 128 or 256).
static void launch_schedule(int bc, bool causal, const FwdParams &p, hipStream_t st) {
    const dim3 g1(1), b1(kSchedThreads);
    if (bc == 64) {
        if (causal) hipLaunchKernelGGL((varlen_schedule_kernel<64, true>), g1, b1, 0, st, p);
        else hipLaunchKernelGGL((varlen_schedule_kernel<64, false>), g1, b1, 0, st, p);
    } else if (bc == 128) {
        if (causal) hipLaunchKernelGGL((varlen_schedule_kernel<128, true>), g1, b1, 0, st, p);
        else hipLaunchKernelGGL((varlen_schedule_kernel<128, false>), g1, b1, 0, st, p);
    } else {
        if (causal) hipLaunchKernelGGL((varlen_schedule_kernel<256, true>), g1, b1, 0, st, p);
        else hipLaunchKernelGGL((varlen_schedule_kernel<256, false>), g1, b1, 0, st, p);
    }
}

hipError_t launch_varlen_schedule(int d, int causal, const int32_t *cu, int num_seqs, int n,
                                  int32_t *sched, int sched_max, int sched_shift, hipStream_t st) {
    FwdParams p{};
    p.cu = cu;
    p.num_seqs = num_seqs;
    p.n_q = n;
    p.sched = sched;
    p.sched_max = sched_max;
    p.sched_shift = sched_shift;
    launch_schedule(fwd16_block_keys(d, 8), causal != 0, p, st);
    return hipGetLastError();
}

// ------------------------------------------------ tile-pruned forward
// TIGA-lang "tile-pruned sparse attention", admission rule: a (128-row,
// 128-key) tile of the dense relation is admitted iff its maximum score reaches
// the query block's running maximum (over admitted tiles) plus ln(rho), with
// p.prune_thr = ln(rho) / scale in raw score units; a pruned tile contributes
// nothing and its V block is never read.
//
// The 8 waves (4 row groups of 32 rows x 2 key groups of 64 keys) run a
// pipeline with one block of lag: in iteration j they score block j+1 and
// exchange the tile maxima through LDS, start V(j+1) only if that tile is
// admitted, and then run the softmax and P.V of block j (if admitted) from the
// scores kept in registers.  K is copied two blocks ahead, V one; each has two
// LDS slots, and one barrier at the top of the iteration (after the copies
// that block j needs have landed) frees the slots the iteration refills.
template <typename T, int D, bool O16>
__device__ __forceinline__ void fwd16_pruned_tile(const FwdParams &p, char *smem, int h, int q_lo,
                                                  int q_hi) {
    constexpr int NST = D == 64 ? 4 : 2;  // the finish routine's view of the LDS
    constexpr int NW = 8, RG = 4, KG = 2, BC = 128, KH = BC / KG, NS = KH / 32;
    static_assert(Fwd16Cfg<D, NST>::BC == BC, "pruning tiles are 128 keys");
    constexpr int ROW = D * 2, TILE = BC * ROW, NKK = D / 16, NDT = D / 32;
    constexpr int NDMA = TILE / (64 * NW * 16);  // 16-byte copies per lane per block
    constexpr int KS = 0, VS = 2 * TILE, XCH = 4 * TILE;  // K slots, V slots, tile maxima
    typedef typename Half8<T>::vec vec8;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rg = wave % RG, kg = wave / RG;
    const int c32 = lane & 31, g = lane >> 5;
    constexpr int esz = (int)sizeof(T);
    const int kv_hi = p.n_k;
    const float c = p.scale_log2;

    // F0: this lane's query row as the B operand (zero past the tile end).
    const int qrow = q_lo + 32 * rg + c32;
    const T *qb = static_cast<const T *>(p.q) + (int64_t)h * p.q_sh + (int64_t)q_lo * p.q_sn;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (int64_t)(q_hi - q_lo) * p.q_sn * esz);
    vec8 qreg[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
        qreg[kk] = __builtin_bit_cast(vec8, bload16(rq, ((32 * rg + c32) * (int)p.q_sn + 16 * kk + 8 * g) * esz));

    // F1: copy i of this wave fills bytes [(NW i + wave) KiB, +1 KiB) of a
    // slot; each lane fetches the global chunk its swizzled LDS place holds.
    // Rows at or past kv_hi arrive as zeros.
    const T *kh = static_cast<const T *>(p.k) + (int64_t)h * p.kv_sh;
    const T *vh = static_cast<const T *>(p.v) + (int64_t)h * p.kv_sh;
    const int kv_sn = (int)p.kv_sn;
    const auto copy_block = [&](const T *base, int b, int slot, bool is_v) {
        const int k0 = b * BC;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (int64_t)k0 * kv_sn, (int64_t)(kv_hi - k0) * kv_sn * esz);
        char *dst = smem + slot;
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const int byte = (NW * i + wave) * 1024 + 16 * lane;
            const int row = byte / ROW, pch = (byte % ROW) / 16;
            const int ch = is_v ? swz_vt<ROW>(row, pch) : swz_k<ROW>(row, pch);
            dma16(r, dst + (NW * i + wave) * 1024, row * kv_sn * esz + ch * 16);
        }
    };

    // F2-F3 for block b: this wave's NS chunks of S^T = K Q^T (tail keys -inf),
    // each chunk's row maximum, and the wave's maximum over its admitted rows.
    const auto scores = [&](int b, f32x16 (&S)[NS], float (&mxc)[NS]) {
        const int kw0 = b * BC + kg * KH;
        const char *sk = smem + KS + (b & 1) * TILE;
        float wmax = kNegInf;
#pragma unroll
        for (int cc = 0; cc < NS; ++cc) {
            mxc[cc] = kNegInf;
            S[cc] = zero_vec<f32x16>();
        }
        if (kw0 < kv_hi) {
#pragma unroll
            for (int cc = 0; cc < NS; ++cc) {
                const int row = kg * KH + 32 * cc + c32;
                const char *krow = sk + row * ROW;
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const vec8 a = *reinterpret_cast<const vec8 *>(krow + swz_k<ROW>(row, 2 * kk + g) * 16);
                    S[cc] = Half8<T>::mma(a, qreg[kk], S[cc]);
                }
                const int kc0 = kw0 + 32 * cc;
                if (kc0 + 32 > kv_hi) {
                    f32x16 Sm[1] = {S[cc]};
                    mask_block<1, false>(Sm, kc0, g, kv_hi, qrow);
                    S[cc] = Sm[0];
                }
                float t[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    t[i] = vmax(vmax(S[cc][4 * i], S[cc][4 * i + 1]), vmax(S[cc][4 * i + 2], S[cc][4 * i + 3]));
                mxc[cc] = xor32_max(vmax(vmax(t[0], t[1]), vmax(t[2], t[3])));
                wmax = vmax(wmax, mxc[cc]);
            }
            if (qrow >= q_hi) wmax = kNegInf;  // rows past the tile end do not count
        }
        return wmax;
    };
    // The tile maximum (all 8 waves' maxima through LDS, one barrier) and the
    // admission decision, the same in every wave.
    float m_blk = kNegInf;  // running maximum of the query block (raw score units)
    const auto admit = [&](float wmax) {
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) wmax = vmax(wmax, __shfl_xor(wmax, off));
        float *slot = reinterpret_cast<float *>(smem + XCH);
        if (lane == 0) slot[wave] = wmax;
        wait_lgkmcnt0();
        bare_barrier();
        float m_tile = slot[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) m_tile = vmax(m_tile, slot[w]);
        const bool ok = m_tile >= m_blk + p.prune_thr;
        if (ok) m_blk = vmax(m_blk, m_tile);
        return ok;
    };

    f32x16 U[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) U[dt] = zero_vec<f32x16>();
    float m_ref = kNegInf, m_true = kNegInf, l_run = 0.f;
    // F4-F6 for an admitted block: lazy reference, probabilities, U += V^T P^T.
    const auto accumulate = [&](int b, const f32x16 (&S)[NS], const float (&mxc)[NS]) {
        const char *sv = smem + VS + (b & 1) * TILE;
#pragma unroll
        for (int cc = 0; cc < NS; ++cc) {
            const float mx = mxc[cc];
            m_true = vmax(m_true, mx);
            if (__any((mx - m_ref) * c > kLazyLog2)) {
                const float m_new = vmax(m_ref, mx);
                const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2((m_ref - m_new) * c);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) U[dt] *= alpha;
                l_run *= alpha;
                m_ref = m_new;
            }
            const float mc = (m_ref == kNegInf) ? 0.f : m_ref * c;
            vec8 P[2];
            float ps = 0.f;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                f32x8 x;
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = fast_exp2(fmaf(S[cc][8 * hf + e], c, -mc));
                ps += ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
                P[hf] = __builtin_convertvector(x, vec8);
            }
            l_run += ps;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int r0 = kg * KH + 32 * cc + 16 * hf + 4 * g + ((lane & 15) >> 2);
                const int cq = lane & 3, hh = (lane >> 4) & 1;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const int ch = 4 * dt + 2 * hh + (cq >> 1);
                    const i16x4 lo = lds_read_tr16(sv + r0 * ROW + swz_vt<ROW>(r0, ch) * 16 + 8 * (cq & 1));
                    const i16x4 hi = lds_read_tr16(sv + (r0 + 8) * ROW + swz_vt<ROW>(r0 + 8, ch) * 16 + 8 * (cq & 1));
                    const vec8 a = __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    U[dt] = Half8<T>::mma(a, P[hf], U[dt]);
                }
            }
        }
    };

    const int nblk = (kv_hi + BC - 1) / BC;
    copy_block(kh, 0, KS, false);
    if (nblk > 1) copy_block(kh, 1, KS + TILE, false);
    if (nblk > 1) wait_vmcnt<NDMA>();  // K(0) (copies complete in order)
    else wait_vmcnt<0>();
    bare_barrier();
    f32x16 Sc[NS];
    float mxc[NS];
    bool adm = admit(scores(0, Sc, mxc));
    if (adm) copy_block(vh, 0, VS, true);
#pragma unroll 1
    for (int j = 0; j < nblk; ++j) {
        // K(j+1) and, if block j is admitted, V(j) have landed for every
        // wave; every wave is past its reads of K(j) and V(j-1).
        wait_vmcnt<0>();
        bare_barrier();
        bool adm_n = false;
        f32x16 Sn[NS];
        float mxn[NS];
        if (j + 1 < nblk) {
            if (j + 2 < nblk) copy_block(kh, j + 2, KS + (j & 1) * TILE, false);
            adm_n = admit(scores(j + 1, Sn, mxn));
            if (adm_n) copy_block(vh, j + 1, VS + ((j + 1) & 1) * TILE, true);
        }
        if (adm && kg * KH + j * BC < kv_hi) accumulate(j, Sc, mxc);
        if (j + 1 < nblk) {
#pragma unroll
            for (int cc = 0; cc < NS; ++cc) {
                Sc[cc] = Sn[cc];
                mxc[cc] = mxn[cc];
            }
        }
        adm = adm_n;
    }
    fwd16_finish<T, D, NST, RG, NW, O16>(p, smem, h, q_hi, -1, wave, lane, qrow, U, m_ref, m_true,
                                         l_run, c);
}

// Tile-pruned dense forward: one 128-row tile per workgroup, 128 x 128 tiles at
// both widths.  The LDS holds the rings of fwd16_pruned_tile and, at the end,
// the key-group merge of the finish routine (which sees it as NST stages).
template <typename T, int D, bool O16>
__global__ void __launch_bounds__(kT16) fwd16_pruned_kernel(FwdParams p) {
    constexpr int NST = D == 64 ? 4 : 2;
    static_assert(Fwd16Cfg<D, NST>::BC == 128, "pruning tiles are 128 keys");
    __shared__ __attribute__((aligned(16))) char smem[NST * Fwd16Cfg<D, NST>::STAGE + 256];
    const int h = blockIdx.x % p.H, tile = blockIdx.x / p.H;
    const int q_lo = tile * kBR, q_hi = min(q_lo + kBR, p.n_q);
    fwd16_pruned_tile<T, D, O16>(p, smem, h, q_lo, q_hi);
}

hipError_t launch_forward_pruned(int dtype, int d, FwdParams p, hipStream_t st) {
    p.n_tiles = (p.n_q + kBR - 1) / kBR;
    const int64_t grid = (int64_t)p.n_tiles * p.H;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 g((unsigned)grid), b(kT16);
    const auto go = [&](auto t, auto dd, auto o16) {
        hipLaunchKernelGGL((fwd16_pruned_kernel<decltype(t), decltype(dd)::value, decltype(o16)::value>),
                           g, b, 0, st, p);
    };
    using D64 = std::integral_constant<int, 64>;
    using D128 = std::integral_constant<int, 128>;
    using F = std::false_type;
    using O = std::true_type;
    if (dtype == 1) {
        if (d == 64) p.o16 ? go(_Float16{}, D64{}, O{}) : go(_Float16{}, D64{}, F{});
        else p.o16 ? go(_Float16{}, D128{}, O{}) : go(_Float16{}, D128{}, F{});
    } else {
        if (d == 64) p.o16 ? go(__bf16{}, D64{}, O{}) : go(__bf16{}, D64{}, F{});
        else p.o16 ? go(__bf16{}, D128{}, O{}) : go(__bf16{}, D128{}, F{});
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------- f32
// MFMA v_mfma_f32_32x32x2_f32.  The contraction slots of K Q^T are assigned so
// that lane half g covers features [g D/2, (g+1) D/2): Q stays in registers and
// K is read in 16-byte vectors.  P stays f32.
// KG = 1: 128-row tiles, each wave 32 rows against all BC keys of a block.
// KG = 4 (dense only): 32-row tiles, each wave a key group of BC keys of every
// 4 BC-key block; the four states merge through LDS at the end, each wave
// merging and storing a quarter of the features.  A grid of 32-row tiles
// fills the device where 128-row tiles would need their keys split over
// workgroups and a combine launch.
template <int D, int BC, int MASK, int KG = 1>
__global__ void __launch_bounds__(kThreads, D == 64 ? 2 : 1) fwd32_kernel(FwdParams p) {
    constexpr bool causal = MASK == kCausal || MASK == kVarlenCausal;
    constexpr int BK = KG * BC;                // keys per block
    constexpr int KCH = D / 4;                 // 16-byte chunks per row
    constexpr int LD = BK * KCH / kThreads;    // chunks per thread per tensor
    constexpr int NS = BC / 32, NDT = D / 32, NQ = D / 2, NJ = D / 8;
    static_assert(LD * kThreads == BK * KCH, "block must split evenly over the threads");
    static_assert(KG == 1 || (KG == 4 && MASK == kDense), "key groups serve the dense relation");

    __shared__ u32x4 sK[BK * KCH];
    __shared__ u32x4 sV[BK * KCH];

    FwdWork w;
    int split = -1;
    if constexpr (MASK == kDense) {
        if (KG == 1 && p.splits > 1) {
            // Split-KV item: key range `split` of one tile, split index slowest.
            const int items = p.H * p.n_tiles;
            split = (int)blockIdx.x / items;
            const int r = (int)blockIdx.x % items;
            w.h = r % p.H;
            w.q_lo = (r / p.H) * kBR;
            w.q_hi = min(w.q_lo + kBR, p.n_q);
            w.ok = w.q_lo < p.n_q;
            w.kv_lo = split * p.split_len;
            w.kv_hi = min(w.kv_lo + p.split_len, p.n_k);
        } else {
            w = fwd_work<MASK>(p, 128 / KG);
        }
    } else {
        w = fwd_work<MASK>(p);
    }
    if (!w.ok) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c32 = lane & 31, g = lane >> 5;
    const int kg = KG == 1 ? 0 : wave;         // key group
    const float *qh = static_cast<const float *>(p.q) + (int64_t)w.h * p.q_sh;
    const float *kh = static_cast<const float *>(p.k) + (int64_t)w.h * p.kv_sh;
    const float *vh = static_cast<const float *>(p.v) + (int64_t)w.h * p.kv_sh;

    const int qrow = w.q_lo + (KG == 1 ? wave * 32 : 0) + c32;
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
    const int nblk = (w.kv_hi - w.kv_lo + BK - 1) / BK;
    const float *sVf = reinterpret_cast<const float *>(sV);

    gload(w.kv_lo);
    for (int kb = 0; kb < nblk; ++kb) {
        const int k0 = w.kv_lo + kb * BK;
        const int kw0 = k0 + kg * BC;          // this wave's first key
        __syncthreads();
        lds_store();
        __syncthreads();
        if (kb + 1 < nblk) gload(k0 + BK);
        if (KG > 1 && kw0 >= w.kv_hi) continue;  // a tail block without this group's keys

        f32x16 S[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            S[s] = zero_vec<f32x16>();
            const u32x4 *krow = &sK[(kg * BC + 32 * s + c32) * KCH];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const f32x4 a = __builtin_bit_cast(f32x4, krow[swz(c32, (D / 8) * g + j)]);
#pragma unroll
                for (int e = 0; e < 4; ++e) S[s] = mma_f32(a[e], qreg[4 * j + e], S[s]);
            }
        }
        if (kw0 + BC > w.kv_hi || (causal && kw0 + BC - 1 > w.q_lo))
            mask_block<NS, causal>(S, kw0, g, w.kv_hi, qrow);
        const float alpha = online_update<NS>(S, m_run, l_run, c);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) U[dt] *= alpha;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kl = kg * BC + 32 * s + acc_row(r, g);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const int d = 32 * dt + c32;
                    const float a = sVf[(kl * KCH + swz(kl, d >> 2)) * 4 + (d & 3)];
                    U[dt] = mma_f32(a, S[s][r], U[dt]);
                }
            }
    }
    if constexpr (KG > 1) {
        // Merge the key groups: every wave leaves (m, l, U) in LDS; wave kg then
        // rescales the KG states of each row to the largest maximum, sums them
        // in group order over its quarter of the features and stores it.
        constexpr int SL = (D / 8) / KG;  // 16-byte feature slots per wave
        static_assert(SL * KG == D / 8 && KG * (D / 8) * 64 * 16 <= (int)sizeof(sK) &&
                          KG * 2 * 64 * 4 <= (int)sizeof(sV),
                      "merge buffers fit in the key and value tiles");
        const float l_tot = l_run + __shfl_xor(l_run, 32);
        __syncthreads();  // every wave is done with the last block
        float *st = reinterpret_cast<float *>(sV);  // (KG, 2, 64) floats: m, l
        f32x4 *su = reinterpret_cast<f32x4 *>(sK);  // (KG, D/8, 64) float4: U
        st[(kg * 2 + 0) * 64 + lane] = m_run;
        st[(kg * 2 + 1) * 64 + lane] = l_tot;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 v = {U[dt][4 * j], U[dt][4 * j + 1], U[dt][4 * j + 2], U[dt][4 * j + 3]};
                su[(kg * (D / 8) + dt * 4 + j) * 64 + lane] = v;
            }
        __syncthreads();
        float M = kNegInf;
#pragma unroll
        for (int k = 0; k < KG; ++k) M = fmaxf(M, st[(k * 2 + 0) * 64 + lane]);
        const float Mu = (M == kNegInf) ? 0.f : M;
        float a[KG];
#pragma unroll
        for (int k = 0; k < KG; ++k) a[k] = fast_exp2((st[(k * 2 + 0) * 64 + lane] - Mu) * c);
        float l = st[1 * 64 + lane] * a[0];
#pragma unroll
        for (int k = 1; k < KG; ++k) l += st[(k * 2 + 1) * 64 + lane] * a[k];
        if (!qok) return;
        const float inv = 1.f / l;
        float *orow = static_cast<float *>(p.o) + (int64_t)w.h * p.o_sh + (int64_t)qrow * p.o_sn;
#pragma unroll
        for (int i = 0; i < SL; ++i) {
            const int sl = kg * SL + i;
            f32x4 acc = su[sl * 64 + lane] * a[0];
#pragma unroll
            for (int k = 1; k < KG; ++k) {
                const f32x4 u = su[(k * (D / 8) + sl) * 64 + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = fmaf(u[e], a[k], acc[e]);
            }
            *reinterpret_cast<f32x4 *>(orow + 32 * (sl >> 2) + 8 * (sl & 3) + 4 * g) = acc * inv;
        }
        if (kg == 0 && g == 0) {
            p.m[(int64_t)w.h * p.n_q + qrow] = M * p.scale;
            p.l[(int64_t)w.h * p.n_q + qrow] = l;
        }
        return;
    }
    if (split >= 0) fwd_partial<NDT>(p, w, split, qrow, g, U, m_run, l_run);
    else fwd_epilogue<NDT>(p, w, qrow, g, U, m_run, l_run);
}

// ------------------------------------------------------------------ launch
template <typename T, int D, int MASK, bool O16>
static void launch_fwd16_o(const FwdParams &p, int grid, hipStream_t st) {
    constexpr bool varlen = MASK == kVarlen || MASK == kVarlenCausal;
    const dim3 g(grid), b(kT16);
    // 128-row tiles: the pipelined 8-wave kernel, one workgroup per CU.  Varlen
    // problems whose sequences average under kWideVarlenRows rows stay on two
    // 4-wave workgroups per CU instead, where one item's start and end overlap
    // the other workgroup's scan (varlen causal, 16384 tokens in 20 sequences,
    // H=8: D=64 fp16 48.9 us there against 58.5 us on the 8-wave kernel, D=128
    // bf16 77.5 against 88.2 us; 6 sequences of 2000-8192 tokens, D=64: 255.6
    // against 232.1 us).
    if (p.tile_rows == kBR && (!varlen || (int64_t)p.n_q >= (int64_t)kWideVarlenRows * p.num_seqs)) {
        hipLaunchKernelGGL((fwd_wide_kernel<T, D, MASK, O16>), g, dim3(64 * WideCfg<D>::NW), 0, st, p);
        return;
    }
    if constexpr (varlen) {
        hipLaunchKernelGGL((fwd16_kernel<T, D, MASK, 2, 4, 4, O16>), g, dim3(256), 0, st, p);
    } else {
        // 64- and (D = 64) 32-row tiles of small dense and causal grids
        if (p.tile_rows == 64) {
            hipLaunchKernelGGL((fwd16_kernel<T, D, MASK, 2, 2, 8, O16>), g, b, 0, st, p);
        } else if constexpr (D == 64) {
            hipLaunchKernelGGL((fwd16_kernel<T, D, MASK, 2, 1, 8, O16>), g, b, 0, st, p);
        }
    }
}

template <typename T, int D, int MASK>
static void launch_fwd16(const FwdParams &p, int grid, hipStream_t st) {
    if (p.o16) launch_fwd16_o<T, D, MASK, true>(p, grid, st);
    else launch_fwd16_o<T, D, MASK, false>(p, grid, st);
}

template <int MASK>
static void launch_fwd_mask(int dtype, int d, const FwdParams &p, int grid16, int grid32,
                            hipStream_t st) {
    if (dtype == 1) {
        if (d == 64) launch_fwd16<_Float16, 64, MASK>(p, grid16, st);
        else launch_fwd16<_Float16, 128, MASK>(p, grid16, st);
    } else if (dtype == 2) {
        if (d == 64) launch_fwd16<__bf16, 64, MASK>(p, grid16, st);
        else launch_fwd16<__bf16, 128, MASK>(p, grid16, st);
    } else {
        if (d == 64 && MASK == kDense && p.f32_groups == 4)
            hipLaunchKernelGGL((fwd32_kernel<64, 32, kDense, 4>), dim3(grid32), dim3(kThreads), 0, st, p);
        else if (d == 64) hipLaunchKernelGGL((fwd32_kernel<64, 64, MASK>), dim3(grid32), dim3(kThreads), 0, st, p);
        else hipLaunchKernelGGL((fwd32_kernel<128, 32, MASK>), dim3(grid32), dim3(kThreads), 0, st, p);
    }
}

// Host entry used by the C ABI (arguments already validated).
hipError_t launch_forward(int dtype, int d, int mask, FwdParams p, int max_seqlen,
                          hipStream_t st) {
    const bool varlen = mask >= kVarlen, causal = mask == kCausal || mask == kVarlenCausal;
    const int rows = varlen ? max_seqlen : p.n_q;
    // 16-bit tiles are p.tile_rows (128, or 64 / 32 for small dense and causal
    // problems); f32 tiles are kBR.
    if (dtype == 0 || varlen || (p.tile_rows != 64 && p.tile_rows != 32)) p.tile_rows = kBR;
    if (dtype == 0 && p.f32_groups == 4) p.tile_rows = 32;  // f32 key groups: 32-row tiles
    if (d != 64 && p.tile_rows == 32) p.tile_rows = 64;
    p.n_tiles = (rows + p.tile_rows - 1) / p.tile_rows;
    const int64_t seqs = varlen ? p.num_seqs : 1;
    // f32 kernel: one workgroup per (head, sequence, tile), times the key
    // splits (dense only).
    const int64_t grid32 = (int64_t)p.n_tiles * p.H * seqs * ((causal || varlen) ? 1 : p.splits);
    // 16-bit kernel: tile pairs for causal / varlen, single tiles otherwise.
    if (!causal || varlen) p.pair = varlen ? 1 : 0;
    const bool paired = p.pair != 0;
    const int64_t grid16 = (int64_t)(paired ? (p.n_tiles + 1) / 2 : p.n_tiles) * p.H * seqs *
                           ((causal || varlen) ? 1 : p.splits);
    if (grid32 <= 0) return hipSuccess;
    if (grid32 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    int64_t g16 = grid16;
    if (p.sched && varlen && dtype != 0) {  // sorted varlen work list first
        // the list's work estimate counts the forward's own key blocks
        launch_schedule(fwd16_block_keys(d, p.waves), causal, p, st);
        g16 = (int64_t)p.sched_max * p.H;
    } else if (p.sched_inline && varlen && dtype != 0 && p.num_seqs <= 64) {
        p.sched = nullptr;
        g16 = (int64_t)p.sched_max * p.H;  // each workgroup ranks its own item
    } else {
        p.sched = nullptr;
        p.sched_inline = 0;
    }
    if (g16 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    switch (mask) {
        case kDense: launch_fwd_mask<kDense>(dtype, d, p, (int)g16, (int)grid32, st); break;
        case kCausal: launch_fwd_mask<kCausal>(dtype, d, p, (int)g16, (int)grid32, st); break;
        case kVarlen: launch_fwd_mask<kVarlen>(dtype, d, p, (int)g16, (int)grid32, st); break;
        default: launch_fwd_mask<kVarlenCausal>(dtype, d, p, (int)g16, (int)grid32, st); break;
    }
    if (p.splits > 1) {  // merge the partial states in a second launch
        const int rows = d == 64 ? kCombineRows<64> : kCombineRows<128>;
        const dim3 gr(p.H * ((p.n_q + rows - 1) / rows)), bl(256);
        if (!p.o16) {
            if (d == 64) hipLaunchKernelGGL((fwd_combine_kernel<64, float>), gr, bl, 0, st, p);
            else hipLaunchKernelGGL((fwd_combine_kernel<128, float>), gr, bl, 0, st, p);
        } else if (dtype == 1) {
            if (d == 64) hipLaunchKernelGGL((fwd_combine_kernel<64, _Float16>), gr, bl, 0, st, p);
            else hipLaunchKernelGGL((fwd_combine_kernel<128, _Float16>), gr, bl, 0, st, p);
        } else {
            if (d == 64) hipLaunchKernelGGL((fwd_combine_kernel<64, __bf16>), gr, bl, 0, st, p);
            else hipLaunchKernelGGL((fwd_combine_kernel<128, __bf16>), gr, bl, 0, st, p);
        }
    }
    return hipGetLastError();
}

}  // namespace osattn
