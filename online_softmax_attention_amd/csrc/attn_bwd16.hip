// Backward attention kernels for gfx950, fp16/bf16 inputs, feature width 64 or
// 128 (v_mfma_f32_32x32x16_{f16,bf16}, f32 accumulation).
//
// Method: OCANNL "Module Ir.Online_softmax", third rewrite bullet (the fused
// backward): a per-row D = sum(dO * O), then nests that recompute each pair's
// p, dp and ds = p * (dp - D) from the forward's row state -- one over the
// query rows accumulating dQ, one over the keys accumulating dK and dV -- each
// owning what it writes.  The mask and the scale act on ds only.  No
// (N_q, N_k) buffer exists at any point.
//
// Row state.  The pre-pass folds m and l into one base-2 offset per row,
// beta = m log2(e) + log2(l), so that p = 2^(s c - beta) with c = scale log2(e)
// (one exponential, no division), next to D.
//
// Kernels (one stream): bwd16_pre, then bwd16_kernel, whose blocks run the
// dK/dV items first and the dQ items after them in the same launch:
//   bwd16_pre  : D_i, beta_i                                             (B0)
//   dK/dV item : a workgroup owns 128 keys, resident in LDS; its 8 waves are
//                4 key groups of 32 keys x 2 query halves, and scan blocks of
//                queries whose Q, dO, beta and D arrive by LDS DMA, two stages
//                deep.  Per 32-query chunk: S = Q K^T, dP = dO V^T (row
//                operands, ds_read_b128), P, dS, then dV^T += dO^T P and
//                dK^T += Q^T dS with the transposed operands read by
//                ds_read_b64_tr_b16; every lane owns one key column.  The two
//                query halves merge through LDS at the end.              (B1)
//   dQ item    : a workgroup owns 128 queries (4 row groups x 2 key halves,
//                one query column per lane) and scans key blocks whose K and V
//                arrive by LDS DMA: S^T = K Q^T, dP^T = V dO^T, P^T, dS^T,
//                dQ^T += K^T dS^T with K^T read transposed.              (B2)
//   reduce     : sums the f32 partials of a split reduction in a fixed order
//                and rounds to the gradient dtype (no atomics).
// Tiles read both as MFMA rows and transposed use the swz_rt swizzle; tiles
// read only as rows use swz_k.
#include "attn_device.h"

namespace osattn {

constexpr int kB16T = 512;  // threads per workgroup (8 waves)

template <int D>
struct Bwd16Cfg {
    static constexpr int ROW = D * 2;   // bytes per 16-bit row
    static constexpr int NKK = D / 16;  // 16-feature slices of the contraction
    static constexpr int NDT = D / 32;  // 32-feature accumulator tiles
    // dQ pass: key blocks of BC keys, K and V double-buffered.
    static constexpr int BC = D == 64 ? 256 : 128;
    static constexpr int KH = BC / 2, NSQ = KH / 32;
    static constexpr int KTILE = BC * ROW;
    static constexpr int KSTAGE = 2 * KTILE;
    static constexpr int NDMA_Q = KTILE / (kB16T * 16);
    // dK/dV pass: BK resident keys, query blocks of BQ double-buffered.
    static constexpr int BK = 128;
    static constexpr int BQ = D == 64 ? 128 : 64;
    static constexpr int QH = BQ / 2, NSK = QH / 32;
    static constexpr int QTILE = BQ * ROW;
    static constexpr int QSTAGE = 2 * QTILE + 2 * BQ * 4;  // Q, dO, beta, D
    static constexpr int KVRES = 2 * BK * ROW;             // resident K, V
    static constexpr int NDMA_K = QTILE / (kB16T * 16);
    static constexpr int NDMA_KV = BK * ROW / (kB16T * 16);
    static constexpr int LDS_DQ = 2 * KSTAGE;
    static constexpr int LDS_DKDV_LOOP = KVRES + 2 * QSTAGE;
    static constexpr int LDS_DKDV_MERGE = 4 * 2 * NDT * 16 * 64 * 4;
    static constexpr int LDS_DKDV = LDS_DKDV_LOOP > LDS_DKDV_MERGE ? LDS_DKDV_LOOP : LDS_DKDV_MERGE;
    static_assert(NDMA_Q * kB16T * 16 == KTILE && NDMA_K * kB16T * 16 == QTILE &&
                      NDMA_KV * kB16T * 16 == BK * ROW,
                  "tiles must split evenly over the DMA lanes");
    static_assert(BQ % 64 == 0, "statistics DMA moves 64 floats per instruction");
};

// ---------------------------------------------------------------- B0
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd16_pre_kernel(BwdParams p) {
    constexpr int PER = D / 16;  // features per thread; 16 threads per row
    const int64_t total = (int64_t)p.H * p.n_q;
    const int64_t row = (int64_t)blockIdx.x * 16 + threadIdx.x / 16;
    const int sub = threadIdx.x % 16;
    float acc = 0.f;
    if (row < total) {
        const int h = (int)(row / p.n_q), i = (int)(row % p.n_q);
        const T *dorow = static_cast<const T *>(p.d_o) + (int64_t)h * p.q_sh + (int64_t)i * p.q_sn;
        const int64_t off = (int64_t)h * p.o_sh + (int64_t)i * p.o_sn + sub * PER;
        if (p.o16) {
            const T *orow = static_cast<const T *>(p.o) + off;
#pragma unroll
            for (int e = 0; e < PER; ++e) acc += (float)dorow[sub * PER + e] * (float)orow[e];
        } else {
            const float *orow = static_cast<const float *>(p.o) + off;
#pragma unroll
            for (int e = 0; e < PER; ++e) acc += (float)dorow[sub * PER + e] * orow[e];
        }
    }
    acc += __shfl_xor(acc, 8);
    acc += __shfl_xor(acc, 4);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 1);
    if (sub == 0 && row < total) {
        p.stat_delta[row] = acc;
        p.stat_mlog2[row] = p.m[row] * kLog2e + __log2f(p.l[row]);  // beta
    }
}

struct Range16 {
    int lo, hi;
};

template <bool VARLEN>
__device__ __forceinline__ Range16 axis16(const BwdParams &p, int seq, int n) {
    if (!VARLEN) return {0, n};
    const Span s = seq_bounds(p.cu, seq, n);
    return {s.lo, s.hi};
}

// Part `split` of [lo, hi) cut into `splits` pieces aligned to `blk`.
__device__ __forceinline__ Range16 split16(int lo, int hi, int split, int splits, int blk) {
    const int len = hi > lo ? hi - lo : 0;
    int chunk = (len + splits - 1) / splits;
    chunk = (chunk + blk - 1) / blk * blk;
    const int a = lo + split * chunk;
    const int b = min(a + chunk, hi);
    return {a, b > a ? b : a};
}

// x, opaque to the optimizer: an address formed from it is formed where it is
// used, not hoisted out of the tile loop into a register held for the whole
// kernel.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// At D = 64 a wave raises its priority for the matrix phases of a chunk and
// drops it for the vector phase in between (s_setprio), which favours the
// wave whose MFMAs are ready over the other wave of its SIMD.  Measured on two
// boxes (same-box interleaved runs, N=4096 H=16 D=64 fp16): causal 1.3-4.1% and
// dense 1.5-1.8% faster, results bit-identical; at D = 128 it moved nothing
// beyond noise, so it stays off there.
template <int D>
__device__ __forceinline__ void prio_matrix() {
    if constexpr (D == 64) __builtin_amdgcn_s_setprio(1);
}
template <int D>
__device__ __forceinline__ void prio_vector() {
    if constexpr (D == 64) __builtin_amdgcn_s_setprio(0);
}

// Store a lane's transposed accumulator tiles (feature rows, one position
// column) as one row of `out`, scaled and rounded to T (or f32 partials).
template <typename T, int NDT>
__device__ __forceinline__ void store_row16(T *rowp, const f32x16 (&acc)[NDT], int g, float scale) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            typedef T t4 __attribute__((ext_vector_type(4)));
            f32x4 v = {acc[dt][4 * j] * scale, acc[dt][4 * j + 1] * scale, acc[dt][4 * j + 2] * scale,
                       acc[dt][4 * j + 3] * scale};
            *reinterpret_cast<t4 *>(rowp + 32 * dt + 8 * j + 4 * g) = __builtin_convertvector(v, t4);
        }
}
// Rows [0, nrows) (at most 32) of a 16-bit output whose row 0 is `rows` (row
// stride sn elements), from a wave's transposed accumulator tiles (lane = row,
// registers = features), scaled and rounded to T.  The values pass through
// `stg` (the wave's own LDS, 32 rows of 2 D + 16 bytes): stored straight from
// the tiles every instruction would write 8 bytes into each of 32 rows, which
// measured ~8K cycles for the 64 KiB of a dK/dV item; from the staging each
// instruction writes whole rows.
template <typename T, int D>
__device__ __forceinline__ void store_rows16_staged(char *stg, T *rows, int64_t sn, int nrows,
                                                    const f32x16 (&acc)[D / 32], float scale, int lane) {
    constexpr int P = 2 * D + 16;  // staging pitch in bytes (16-byte aligned rows)
    typedef T t4 __attribute__((ext_vector_type(4)));
    const int c32 = lane & 31, g = lane >> 5;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4 v = {acc[dt][4 * j] * scale, acc[dt][4 * j + 1] * scale, acc[dt][4 * j + 2] * scale,
                       acc[dt][4 * j + 3] * scale};
            *reinterpret_cast<t4 *>(stg + c32 * P + (32 * dt + 8 * j + 4 * g) * 2) = __builtin_convertvector(v, t4);
        }
    wait_lgkmcnt0();
    asm volatile("" ::: "memory");
    constexpr int LPR = 2 * D / 16, RPI = 64 / LPR;  // lanes per row, rows per instruction
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
        const int r = RPI * i + lane / LPR, c = lane % LPR;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(stg + r * P + 16 * c);
        if (r < nrows) *reinterpret_cast<u32x4 *>(rows + (int64_t)r * sn + 8 * c) = v;
    }
}

template <int NDT>
__device__ __forceinline__ void store_row_part(float *rowp, const f32x16 (&acc)[NDT], int g, float scale) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4 v = {acc[dt][4 * j] * scale, acc[dt][4 * j + 1] * scale, acc[dt][4 * j + 2] * scale,
                       acc[dt][4 * j + 3] * scale};
            *reinterpret_cast<f32x4 *>(rowp + 32 * dt + 8 * j + 4 * g) = v;
        }
}

// A operand of a transposed product: rows [r0, r0 + 4) and [r0 + 8, r0 + 12)
// of a row-major 16-bit tile (swz_rt), feature chunk ch, as 8 values per lane.
template <typename T, int ROW>
__device__ __forceinline__ typename Half8<T>::vec tr_operand(const char *tile, int r0, int ch, int cq) {
    const i16x4 lo = lds_read_tr16(tile + r0 * ROW + swz_rt<ROW>(r0, ch) * 16 + 8 * (cq & 1));
    const i16x4 hi = lds_read_tr16(tile + (r0 + 8) * ROW + swz_rt<ROW>(r0 + 8, ch) * 16 + 8 * (cq & 1));
    return __builtin_bit_cast(typename Half8<T>::vec, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---------------------------------------------------------------- B1
// One 128-key tile: keys [k_lo, min(k_lo + 128, ks.hi)) against the queries
// of qs_all (from k_lo on when causal), part `split` of k_splits.
template <typename T, int D, int MASK>
__device__ __forceinline__ void dkdv16_tile(const BwdParams &p, char *smem, int h, int split,
                                            Range16 ks, Range16 qs_all, int k_lo) {
    typedef Bwd16Cfg<D> C;
    typedef typename Half8<T>::vec vec8;
    constexpr bool causal = MASK == kCausal || MASK == kVarlenCausal;
    constexpr bool varlen = MASK == kVarlen || MASK == kVarlenCausal;
    constexpr int esz = (int)sizeof(T);
    const int k_hi = min(k_lo + C::BK, ks.hi);
    const int qa = causal ? max(qs_all.lo, k_lo) : qs_all.lo;
    const Range16 qr = split16(qa, qs_all.hi, split, p.k_splits, C::BQ);

    // The wave index is uniform; taking it into a scalar register makes the
    // per-wave tests below (tail, diagonal chunk) scalar branches instead of
    // masked selects on every element.
    const int tid = threadIdx.x, lane = opaque(tid & 63), wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kq = wave & 3, qg = wave >> 2;  // key group, query half
    const int c32 = lane & 31, g = lane >> 5;
    const int key = k_lo + 32 * kq + c32;      // this lane's key column
    const int kv_sn = (int)p.kv_sn, q_sn = (int)p.q_sn;

    // Resident K and V of the tile (rows past k_hi arrive as zeros).  The
    // copies are inline assembly (dma16_asm): the compiler, which would make
    // the transposed operand reads of a block wait for the next block's copy
    // in flight, leaves their order to the explicit waits and barriers, and
    // the compiler's fences no longer wait for them either.  A tile with no
    // query block (an empty part of a split query range) copies nothing: its
    // merge writes this LDS at once.
    char *sK = smem, *sV = smem + C::BK * C::ROW;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(OSATTN_LDS char *)smem;
    const int nblk = (qr.hi - qr.lo + C::BQ - 1) / C::BQ;
    if (nblk > 0) {
        const T *kb = static_cast<const T *>(p.k) + (int64_t)h * p.kv_sh + (int64_t)k_lo * p.kv_sn;
        const T *vb = static_cast<const T *>(p.v) + (int64_t)h * p.kv_sh + (int64_t)k_lo * p.kv_sn;
        const int64_t bytes = (int64_t)(k_hi - k_lo) * p.kv_sn * esz;
        const i32x4 rk = rsrc_words64(kb, bytes), rv = rsrc_words64(vb, bytes);
#pragma unroll
        for (int i = 0; i < C::NDMA_KV; ++i) {
            const int byte = (8 * i + wave) * 1024 + 16 * lane;
            const int row = byte / C::ROW, pch = (byte % C::ROW) / 16;
            const int off = row * kv_sn * esz + swz_k<C::ROW>(row, pch) * 16;
            dma16_asm(rk, lds0 + (8 * i + wave) * 1024, off);
            dma16_asm(rv, lds0 + C::BK * C::ROW + (8 * i + wave) * 1024, off);
        }
    }

    // Query block DMA into stage `buf`: Q and dO rows (swz_rt), beta and D.
    const T *qh = static_cast<const T *>(p.q) + (int64_t)h * p.q_sh;
    const T *doh = static_cast<const T *>(p.d_o) + (int64_t)h * p.q_sh;
    const float *bh = p.stat_mlog2 + (int64_t)h * p.n_q;
    const float *dh = p.stat_delta + (int64_t)h * p.n_q;
    char *stage0 = smem + C::KVRES;
    auto issue = [&](int q0, int buf) {
        const uint32_t sq = lds0 + C::KVRES + buf * C::QSTAGE;
        const uint32_t sdo = sq + C::QTILE;
        const uint32_t sb = sdo + C::QTILE;  // beta, then D
        const uint32_t sd = sb + 4 * C::BQ;
        const int64_t bytes = (int64_t)(qr.hi - q0) * p.q_sn * esz;
        const i32x4 rq = rsrc_words64(qh + (int64_t)q0 * p.q_sn, bytes);
        const i32x4 rd = rsrc_words64(doh + (int64_t)q0 * p.q_sn, bytes);
#pragma unroll
        for (int i = 0; i < C::NDMA_K; ++i) {
            const int byte = (8 * i + wave) * 1024 + 16 * lane;
            const int row = byte / C::ROW, pch = (byte % C::ROW) / 16;
            const int off = row * q_sn * esz + swz_rt<C::ROW>(row, pch) * 16;
            dma16_asm(rq, sq + (8 * i + wave) * 1024, off);
            dma16_asm(rd, sdo + (8 * i + wave) * 1024, off);
        }
        // beta and D: waves 0 .. BQ/64 - 1 move 64 floats each per array.
        if (wave < C::BQ / 64) {
            const int64_t sbytes = (int64_t)(qr.hi - q0) * 4;
            const i32x4 rb = rsrc_words64(bh + q0, sbytes), rdl = rsrc_words64(dh + q0, sbytes);
            dma4_asm(rb, sb + 256 * wave, 4 * (64 * wave + lane));
            dma4_asm(rdl, sd + 256 * wave, 4 * (64 * wave + lane));
        }
    };

    f32x16 dK[C::NDT], dV[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
        dK[dt] = zero_vec<f32x16>();
        dV[dt] = zero_vec<f32x16>();
    }
    const float c = p.scale_log2;
    const int krow = 32 * kq + c32;  // this lane's row of the resident tiles

    if (nblk > 0) issue(qr.lo, 0);
    for (int j = 0; j < nblk; ++j) {
        // Block j (and, for j = 0, the resident K/V) has landed for this
        // thread, and after the barrier for all; block j-1's stage is free.
        wait_vmcnt<0>();
        bare_barrier();
        if (j + 1 < nblk) issue(qr.lo + (j + 1) * C::BQ, (j + 1) & 1);

        const int q0 = qr.lo + j * C::BQ;
        const char *sq = stage0 + (j & 1) * C::QSTAGE;
        const char *sdo = sq + C::QTILE;
        const float *sb = reinterpret_cast<const float *>(sdo + C::QTILE);
        const float *sd = sb + C::BQ;
#pragma unroll
        for (int cc = 0; cc < C::NSK; ++cc) {
            const int ql0 = qg * C::QH + 32 * cc;  // chunk's first row in the block
            const int qc0 = q0 + ql0;
            if (qc0 >= qr.hi) break;
            if (causal && k_lo + 32 * kq > qc0 + 31) continue;  // every pair masked
            // S = Q K^T and dP = dO V^T: rows = the chunk's queries, column =
            // this lane's key.  The two chains alternate so that each one's
            // LDS reads are in flight while the other's MFMA runs.
            f32x16 S = zero_vec<f32x16>(), dP = zero_vec<f32x16>();
            const int qrow = ql0 + c32;
            prio_matrix<D>();
#pragma unroll
            for (int kk = 0; kk < C::NKK; ++kk) {
                const vec8 qa8 = *reinterpret_cast<const vec8 *>(sq + qrow * C::ROW + swz_rt<C::ROW>(qrow, 2 * kk + g) * 16);
                const vec8 kb8 = *reinterpret_cast<const vec8 *>(sK + krow * C::ROW + swz_k<C::ROW>(krow, 2 * kk + g) * 16);
                const vec8 da8 = *reinterpret_cast<const vec8 *>(sdo + qrow * C::ROW + swz_rt<C::ROW>(qrow, 2 * kk + g) * 16);
                const vec8 vb8 = *reinterpret_cast<const vec8 *>(sV + krow * C::ROW + swz_k<C::ROW>(krow, 2 * kk + g) * 16);
                S = Half8<T>::mma(qa8, kb8, S);
                dP = Half8<T>::mma(da8, vb8, dP);
            }
            prio_vector<D>();
            // P = 2^(s c - beta), zero where key > query; dS = P (dP - D).
            if (causal && k_lo + 32 * kq + 31 > qc0) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (key > qc0 + acc_row(r, g)) S[r] = kNegInf;
            }
            f32x16 P, dS;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 bv = *reinterpret_cast<const f32x4 *>(sb + ql0 + 8 * i + 4 * g);
                const f32x4 dv = *reinterpret_cast<const f32x4 *>(sd + ql0 + 8 * i + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * i + e;
                    const float pv = fast_exp2(fmaf(S[r], c, -bv[e]));
                    P[r] = pv;
                    dS[r] = pv * (dP[r] - dv[e]);
                }
            }
            // dV^T += dO^T P and dK^T += Q^T dS over the chunk's two 16-query
            // slices; slice hf holds rows 16 hf + 8 x + 4 g + 0..3 (x = 0, 1).
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                f32x8 pp, ss;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pp[e] = P[8 * hf + e];
                    ss[e] = dS[8 * hf + e];
                }
                const vec8 pb = __builtin_convertvector(pp, vec8);
                const vec8 sbv = __builtin_convertvector(ss, vec8);
                const int r0 = ql0 + 16 * hf + 4 * g + ((lane & 15) >> 2);
                const int cq = lane & 3, hh = (lane >> 4) & 1;
                prio_matrix<D>();
#pragma unroll
                for (int dt = 0; dt < C::NDT; ++dt) {
                    const int ch = 4 * dt + 2 * hh + (cq >> 1);
                    dV[dt] = Half8<T>::mma(tr_operand<T, C::ROW>(sdo, r0, ch, cq), pb, dV[dt]);
                    dK[dt] = Half8<T>::mma(tr_operand<T, C::ROW>(sq, r0, ch, cq), sbv, dK[dt]);
                }
            }
        }
    }
    prio_vector<D>();
    wait_vmcnt<0>();  // no copy is in flight (each was waited for in the loop)
    __syncthreads();  // every wave is done with the stages and the resident tiles

    // Merge the two query halves: half 1 leaves dK^T, dV^T in LDS.
    f32x4 *sm = reinterpret_cast<f32x4 *>(smem);  // (4 key groups, 2, D/8, 64) float4
    if (qg == 1) {
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                f32x4 a = {dK[dt][4 * jj], dK[dt][4 * jj + 1], dK[dt][4 * jj + 2], dK[dt][4 * jj + 3]};
                f32x4 v = {dV[dt][4 * jj], dV[dt][4 * jj + 1], dV[dt][4 * jj + 2], dV[dt][4 * jj + 3]};
                sm[((kq * 2 + 0) * (D / 8) + dt * 4 + jj) * 64 + lane] = a;
                sm[((kq * 2 + 1) * (D / 8) + dt * 4 + jj) * 64 + lane] = v;
            }
    }
    __syncthreads();
    if (qg == 0) {
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const f32x4 a = sm[((kq * 2 + 0) * (D / 8) + dt * 4 + jj) * 64 + lane];
                const f32x4 v = sm[((kq * 2 + 1) * (D / 8) + dt * 4 + jj) * 64 + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dK[dt][4 * jj + e] += a[e];
                    dV[dt][4 * jj + e] += v[e];
                }
            }
        if (varlen || p.k_splits == 1) {  // varlen keys are never split
            // The staging reuses this wave's own half of the merge buffer,
            // once every read of it has returned.
            wait_lgkmcnt0();
            asm volatile("" ::: "memory");
            char *stg = smem + kq * 2 * (D / 8) * 64 * 16;
            const int r0 = k_lo + 32 * kq;
            const int64_t koff = (int64_t)h * p.kv_sh + (int64_t)opaque(r0) * p.kv_sn;
            store_rows16_staged<T, D>(stg, static_cast<T *>(p.dk) + koff, p.kv_sn, k_hi - r0, dK, p.scale, lane);
            store_rows16_staged<T, D>(stg + 32 * (2 * D + 16), static_cast<T *>(p.dv) + koff, p.kv_sn,
                                      k_hi - r0, dV, 1.f, lane);
        } else if (key < k_hi) {
            const int64_t off = (((int64_t)split * p.H + h) * p.n_k + key) * D;
            store_row_part<C::NDT>(p.dk_part + off, dK, g, p.scale);
            store_row_part<C::NDT>(p.dv_part + off, dV, g, 1.f);
        }
    }
    __syncthreads();  // the next tile reuses this LDS
}

// Work item b of the dK/dV pass.  SCHED: varlen items from the sorted work
// list (one or two tiles each); otherwise one tile of the natural grid, or
// with pair_k (causal) the tiles i and T-1-i, T-i and i+1 query tiles of work.
template <typename T, int D, int MASK, bool SCHED>
__device__ __forceinline__ void dkdv16_item(const BwdParams &p, char *smem, int b) {
    constexpr bool varlen = MASK == kVarlen || MASK == kVarlenCausal;
    const int h = b % p.H;
    int rest = b / p.H;
    // The item: a key range [lo, hi) with up to two 128-key tiles of it, and
    // the query range [qlo, qhi) those keys meet.
    int split = 0, lo, hi, qlo, qhi, t0, t1 = -1;
    if constexpr (SCHED) {  // tiles (T-1-i, i) of one sequence, largest pairs first
        // uniform: taken into scalar registers
        const int4 it = reinterpret_cast<const int4 *>(p.sched + 4)[rest];
        lo = qlo = __builtin_amdgcn_readfirstlane(it.x);
        hi = qhi = __builtin_amdgcn_readfirstlane(it.y);
        t0 = __builtin_amdgcn_readfirstlane(it.z);
        t1 = __builtin_amdgcn_readfirstlane(it.w);
    } else {
        split = rest % p.k_splits;
        rest /= p.k_splits;
        int seq = 0;
        if (varlen) {
            seq = rest % p.num_seqs;
            rest /= p.num_seqs;
        }
        const Range16 ks = axis16<varlen>(p, seq, p.n_k), qs = axis16<varlen>(p, seq, p.n_q);
        lo = ks.lo; hi = ks.hi; qlo = qs.lo; qhi = qs.hi;
        t0 = rest;  // causal: key tile 0 (the most queries) first
        if (MASK == kCausal && p.pair_k && p.k_tiles - 1 - rest != rest) t1 = p.k_tiles - 1 - rest;
    }
#pragma unroll 1
    for (int k = 0; k < 2; ++k) {
        const int t = k == 0 ? t0 : t1;
        if (t < 0 || lo + t * 128 >= hi) break;
        dkdv16_tile<T, D, MASK>(p, smem, h, split, {lo, hi}, {qlo, qhi}, lo + t * 128);
    }
}

// ---------------------------------------------------------------- B2
// One 128-query tile: rows [q_lo, min(q_lo + 128, qs_all.hi)) against the keys
// of ks_all (up to the tile end when causal), part `split` of q_splits.
template <typename T, int D, int MASK>
__device__ __forceinline__ void dq16_tile(const BwdParams &p, char *smem, int h, int split,
                                          Range16 qs_all, Range16 ks_all, int q_lo) {
    typedef Bwd16Cfg<D> C;
    typedef typename Half8<T>::vec vec8;
    constexpr bool causal = MASK == kCausal || MASK == kVarlenCausal;
    constexpr bool varlen = MASK == kVarlen || MASK == kVarlenCausal;
    constexpr int esz = (int)sizeof(T);
    const int q_hi = min(q_lo + 128, qs_all.hi);
    const int kv_end = causal ? q_hi : ks_all.hi;
    const Range16 kr = split16(ks_all.lo, kv_end, split, p.q_splits, C::BC);
    const int kv_lo = kr.lo, kv_hi = kr.hi;

    const int tid = threadIdx.x, lane = opaque(tid & 63), wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
    const int rg = wave & 3, kg = wave >> 2;
    const int c32 = lane & 31, g = lane >> 5;
    const int qrow = q_lo + 32 * rg + c32;
    const bool qok = qrow < q_hi;

    // This lane's query row of Q and dO as B operands, and its row state.
    const T *qb = static_cast<const T *>(p.q) + (int64_t)h * p.q_sh + (int64_t)q_lo * p.q_sn;
    const T *db = static_cast<const T *>(p.d_o) + (int64_t)h * p.q_sh + (int64_t)q_lo * p.q_sn;
    const int64_t qbytes = (int64_t)(q_hi - q_lo) * p.q_sn * esz;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, qbytes), rdo = make_rsrc(db, qbytes);
    vec8 qreg[C::NKK], doreg[C::NKK];
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
        const int off = ((32 * rg + c32) * (int)p.q_sn + 16 * kk + 8 * g) * esz;
        qreg[kk] = __builtin_bit_cast(vec8, bload16(rq, off));
        doreg[kk] = __builtin_bit_cast(vec8, bload16(rdo, off));
    }
    const int64_t srow = (int64_t)h * p.n_q + qrow;
    const float beta = qok ? p.stat_mlog2[srow] : 0.f;
    const float dl = qok ? p.stat_delta[srow] : 0.f;

    const T *kh = static_cast<const T *>(p.k) + (int64_t)h * p.kv_sh;
    const T *vh = static_cast<const T *>(p.v) + (int64_t)h * p.kv_sh;
    const int kv_sn = (int)p.kv_sn;
    // K and V copies as inline assembly (see dkdv16_tile).
    const uint32_t lds0 = (uint32_t)(uintptr_t)(OSATTN_LDS char *)smem;
    auto issue = [&](int k0, int buf) {
        const int64_t bytes = (int64_t)(kv_hi - k0) * kv_sn * esz;
        const i32x4 rk = rsrc_words64(kh + (int64_t)k0 * kv_sn, bytes);
        const i32x4 rv = rsrc_words64(vh + (int64_t)k0 * kv_sn, bytes);
        const uint32_t sk = lds0 + buf * C::KSTAGE;
        const uint32_t sv = sk + C::KTILE;
#pragma unroll
        for (int i = 0; i < C::NDMA_Q; ++i) {
            const int byte = (8 * i + wave) * 1024 + 16 * lane;
            const int row = byte / C::ROW, pch = (byte % C::ROW) / 16;
            dma16_asm(rk, sk + (8 * i + wave) * 1024, row * kv_sn * esz + swz_rt<C::ROW>(row, pch) * 16);
            dma16_asm(rv, sv + (8 * i + wave) * 1024, row * kv_sn * esz + swz_k<C::ROW>(row, pch) * 16);
        }
    };

    f32x16 dQ[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) dQ[dt] = zero_vec<f32x16>();
    const float c = p.scale_log2;
    const int nblk = (kv_hi - kv_lo + C::BC - 1) / C::BC;
    const int wrow_lo = q_lo + 32 * rg, wrow_hi = wrow_lo + 31;

    if (nblk > 0) issue(kv_lo, 0);
    for (int j = 0; j < nblk; ++j) {
        wait_vmcnt<0>();
        bare_barrier();
        if (j + 1 < nblk) issue(kv_lo + (j + 1) * C::BC, (j + 1) & 1);

        const int k0 = kv_lo + j * C::BC;
        const int kw0 = k0 + kg * C::KH;
        const char *sk = smem + (j & 1) * C::KSTAGE;
        const char *sv = sk + C::KTILE;
        if (kw0 < kv_hi && (!causal || kw0 <= wrow_hi)) {
#pragma unroll
            for (int cc = 0; cc < C::NSQ; ++cc) {
                const int kc0 = kw0 + 32 * cc;
                if (kc0 >= kv_hi || (causal && kc0 > wrow_hi)) break;
                const int row = kg * C::KH + 32 * cc + c32;
                // S^T = K Q^T and dP^T = V dO^T: rows = the chunk's keys,
                // column = this lane's query.
                f32x16 S = zero_vec<f32x16>(), dP = zero_vec<f32x16>();
                prio_matrix<D>();
#pragma unroll
                for (int kk = 0; kk < C::NKK; ++kk) {
                    const vec8 ka = *reinterpret_cast<const vec8 *>(sk + row * C::ROW + swz_rt<C::ROW>(row, 2 * kk + g) * 16);
                    const vec8 va = *reinterpret_cast<const vec8 *>(sv + row * C::ROW + swz_k<C::ROW>(row, 2 * kk + g) * 16);
                    S = Half8<T>::mma(ka, qreg[kk], S);
                    dP = Half8<T>::mma(va, doreg[kk], dP);
                }
                prio_vector<D>();
                if (kc0 + 32 > kv_hi || (causal && kc0 + 31 > wrow_lo)) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {  // tail keys and keys past the diagonal
                        const int kk2 = kc0 + acc_row(r, g);
                        if (kk2 >= kv_hi || (causal && kk2 > qrow)) S[r] = kNegInf;
                    }
                }
                // dS^T = P^T (dP^T - D), P^T = 2^(s c - beta).
                vec8 dsv[2];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    f32x8 x;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float pv = fast_exp2(fmaf(S[8 * hf + e], c, -beta));
                        x[e] = pv * (dP[8 * hf + e] - dl);
                    }
                    dsv[hf] = __builtin_convertvector(x, vec8);
                }
                // dQ^T += K^T dS^T over the chunk's two 16-key slices.
                prio_matrix<D>();
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int r0 = kg * C::KH + 32 * cc + 16 * hf + 4 * g + ((lane & 15) >> 2);
                    const int cq = lane & 3, hh = (lane >> 4) & 1;
#pragma unroll
                    for (int dt = 0; dt < C::NDT; ++dt) {
                        const int ch = 4 * dt + 2 * hh + (cq >> 1);
                        dQ[dt] = Half8<T>::mma(tr_operand<T, C::ROW>(sk, r0, ch, cq), dsv[hf], dQ[dt]);
                    }
                }
            }
        }
    }
    prio_vector<D>();
    wait_vmcnt<0>();  // no copy is in flight (each was waited for in the loop)
    __syncthreads();

    // Merge the two key halves: half 1 leaves dQ^T in LDS.
    f32x4 *sm = reinterpret_cast<f32x4 *>(smem);  // (4 row groups, D/8, 64) float4
    if (kg == 1) {
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                f32x4 a = {dQ[dt][4 * jj], dQ[dt][4 * jj + 1], dQ[dt][4 * jj + 2], dQ[dt][4 * jj + 3]};
                sm[(rg * (D / 8) + dt * 4 + jj) * 64 + lane] = a;
            }
    }
    __syncthreads();
    if (kg == 0) {
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const f32x4 a = sm[(rg * (D / 8) + dt * 4 + jj) * 64 + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) dQ[dt][4 * jj + e] += a[e];
            }
        if (varlen || p.q_splits == 1) {  // varlen queries are never split
            // staged through this wave's own part of the merge buffer
            wait_lgkmcnt0();
            asm volatile("" ::: "memory");
            char *stg = smem + rg * (D / 8) * 64 * 16;
            const int r0 = q_lo + 32 * rg;
            store_rows16_staged<T, D>(stg, static_cast<T *>(p.dq) + (int64_t)h * p.q_sh + (int64_t)opaque(r0) * p.q_sn,
                                      p.q_sn, q_hi - r0, dQ, p.scale, lane);
        } else if (qok) {
            const int64_t off = (((int64_t)split * p.H + h) * p.n_q + qrow) * D;
            store_row_part<C::NDT>(p.dq_part + off, dQ, g, p.scale);
        }
    }
    __syncthreads();  // the next tile reuses this LDS
}

// Work item b of the dQ pass, numbered like the dK/dV items.
template <typename T, int D, int MASK, bool SCHED>
__device__ __forceinline__ void dq16_item(const BwdParams &p, char *smem, int b) {
    constexpr bool causal = MASK == kCausal || MASK == kVarlenCausal;
    constexpr bool varlen = MASK == kVarlen || MASK == kVarlenCausal;
    const int h = b % p.H;
    int rest = b / p.H;
    // The item: a query range [lo, hi) with up to two 128-query tiles of it,
    // and the key range [klo, khi) those queries meet.
    int split = 0, lo, hi, klo, khi, t0, t1 = -1;
    if constexpr (SCHED) {  // tiles (T-1-i, i) of one sequence, largest pairs first
        const int4 it = reinterpret_cast<const int4 *>(p.sched + 4)[rest];
        lo = klo = __builtin_amdgcn_readfirstlane(it.x);
        hi = khi = __builtin_amdgcn_readfirstlane(it.y);
        t0 = __builtin_amdgcn_readfirstlane(it.z);
        t1 = __builtin_amdgcn_readfirstlane(it.w);
    } else {
        split = rest % p.q_splits;
        rest /= p.q_splits;
        int seq = 0;
        if (varlen) {
            seq = rest % p.num_seqs;
            rest /= p.num_seqs;
        }
        const Range16 qs = axis16<varlen>(p, seq, p.n_q), ks = axis16<varlen>(p, seq, p.n_k);
        lo = qs.lo; hi = qs.hi; klo = ks.lo; khi = ks.hi;
        t0 = causal ? (p.q_tiles - 1 - rest) : rest;  // causal: heaviest first
        if (MASK == kCausal && p.pair_q && p.q_tiles - 1 - rest != rest) t1 = rest;
    }
#pragma unroll 1
    for (int k = 0; k < 2; ++k) {
        const int t = k == 0 ? t0 : t1;
        if (t < 0 || lo + t * 128 >= hi) break;
        dq16_tile<T, D, MASK>(p, smem, h, split, {lo, hi}, {klo, khi}, lo + t * 128);
    }
}

// One launch for both passes: blocks [0, grid_k) take the dK/dV items, the
// rest the dQ items.  The two passes write disjoint outputs and read only
// what the pre-pass wrote, so dQ items start on the CUs that the dK/dV tail
// leaves idle instead of waiting for the whole dK/dV grid to drain.
template <typename T, int D, int MASK, bool SCHED>
__global__ void __launch_bounds__(kB16T) bwd16_kernel(BwdParams p) {
    typedef Bwd16Cfg<D> C;
    constexpr int LDS = C::LDS_DKDV > C::LDS_DQ ? C::LDS_DKDV : C::LDS_DQ;
    __shared__ __attribute__((aligned(16))) char smem[LDS];
    const int b = blockIdx.x;
    if (b < p.grid_k)
        dkdv16_item<T, D, MASK, SCHED>(p, smem, b);
    else
        dq16_item<T, D, MASK, SCHED>(p, smem, b - p.grid_k);
}

// ---------------------------------------------------------------- reduce
// Up to three split reductions in one launch (Reduce3), each thread one float4
// of its output summed over the splits in a fixed order, rounded once.
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd16_reduce_kernel(Reduce3 q) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    int64_t b = blockIdx.x;
    const ReduceParams &r = q.r[q.which(b)];
    const int64_t total4 = (int64_t)r.H * r.n * D / 4;
    const int64_t i4 = b * 256 + threadIdx.x;
    if (i4 >= total4) return;
    const int64_t e = i4 * 4;
    const int64_t plane = (int64_t)r.n * D;
    const int h = (int)(e / plane);
    const int64_t rem = e % plane;
    const int i = (int)(rem / D), d = (int)(rem % D);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int64_t stride = (int64_t)r.H * plane;
#pragma unroll 8
    for (int s = 0; s < r.splits; ++s) acc += *reinterpret_cast<const f32x4 *>(r.part + s * stride + e);
    *reinterpret_cast<t4 *>(static_cast<T *>(r.out) + (int64_t)h * r.out_sh + (int64_t)i * r.out_sn + d) =
        __builtin_convertvector(acc, t4);
}

// ------------------------------------------------------------------ launch
template <typename T, int D, int MASK>
static void launch_bwd16_mask(const BwdParams &p, int grid, hipStream_t st) {
    constexpr bool varlen = MASK == kVarlen || MASK == kVarlenCausal;
    if (grid <= 0) return;
    if (varlen && p.sched)
        hipLaunchKernelGGL((bwd16_kernel<T, D, MASK, varlen>), dim3(grid), dim3(kB16T), 0, st, p);
    else
        hipLaunchKernelGGL((bwd16_kernel<T, D, MASK, false>), dim3(grid), dim3(kB16T), 0, st, p);
}

hipError_t launch_varlen_schedule(int d, int causal, const int32_t *cu, int num_seqs, int n,
                                  int32_t *sched, int sched_max, int sched_shift, hipStream_t st);

template <typename T, int D>
static hipError_t launch_bwd16_typed(int mask, const BwdParams &p, int seqs, hipStream_t st) {
    const int64_t rows = (int64_t)p.H * p.n_q;
    hipLaunchKernelGGL((bwd16_pre_kernel<T, D>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // Tile pairs only where the items read them: the causal relation, one split.
    const int pair_k = p.pair_k && mask == kCausal && p.k_splits == 1;
    const int pair_q = p.pair_q && mask == kCausal && p.q_splits == 1;
    int64_t grid_k = (int64_t)p.H * p.k_splits * seqs * (pair_k ? (p.k_tiles + 1) / 2 : p.k_tiles);
    int64_t grid_q = (int64_t)p.H * p.q_splits * seqs * (pair_q ? (p.q_tiles + 1) / 2 : p.q_tiles);
    if (p.sched) grid_k = grid_q = (int64_t)p.H * p.sched_max;  // one workgroup per listed pair
    if (grid_k + grid_q > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    BwdParams pf = p;
    pf.pair_k = pair_k;
    pf.pair_q = pair_q;
    pf.grid_k = (int)grid_k;
    const int grid = (int)(grid_k + grid_q);
    switch (mask) {
        case kDense: launch_bwd16_mask<T, D, kDense>(pf, grid, st); break;
        case kCausal: launch_bwd16_mask<T, D, kCausal>(pf, grid, st); break;
        case kVarlen: launch_bwd16_mask<T, D, kVarlen>(pf, grid, st); break;
        default: launch_bwd16_mask<T, D, kVarlenCausal>(pf, grid, st); break;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // One launch for every split reduction, not one per gradient.
    Reduce3 q{};
    const auto add = [&](const float *part, void *out, int64_t sh, int64_t sn, int n, int splits) {
        const int64_t grid = ((int64_t)p.H * n * D / 4 + 255) / 256;
        if (grid <= 0) return;
        q.r[q.count] = ReduceParams{part, out, sh, sn, p.H, n, splits};
        q.end[q.count] = (q.count ? q.end[q.count - 1] : 0) + grid;
        ++q.count;
    };
    if (p.k_splits > 1) {
        add(p.dk_part, p.dk, p.kv_sh, p.kv_sn, p.n_k, p.k_splits);
        add(p.dv_part, p.dv, p.kv_sh, p.kv_sn, p.n_k, p.k_splits);
    }
    if (p.q_splits > 1) add(p.dq_part, p.dq, p.q_sh, p.q_sn, p.n_q, p.q_splits);
    if (q.count > 0) {
        if (q.end[q.count - 1] > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((bwd16_reduce_kernel<T, D>), dim3((unsigned)q.end[q.count - 1]), dim3(256), 0, st, q);
    }
    return hipGetLastError();
}

// Host entry for fp16/bf16 (dtype 1 / 2), d = 64 or 128 (validated by the ABI).
// With p.sched set (varlen), the work list is written first.
hipError_t launch_backward16(int dtype, int d, int mask, BwdParams p, int seqs, int sched_shift,
                             hipStream_t st) {
    if (p.sched) {
        const hipError_t e = launch_varlen_schedule(d, mask == kVarlenCausal, p.cu, p.num_seqs, p.n_q,
                                                    const_cast<int32_t *>(p.sched), p.sched_max,
                                                    sched_shift, st);
        if (e != hipSuccess) return e;
    }
    if (dtype == 1)
        return d == 64 ? launch_bwd16_typed<_Float16, 64>(mask, p, seqs, st)
                       : launch_bwd16_typed<_Float16, 128>(mask, p, seqs, st);
    return d == 64 ? launch_bwd16_typed<__bf16, 64>(mask, p, seqs, st)
                   : launch_bwd16_typed<__bf16, 128>(mask, p, seqs, st);
}

}  // namespace osattn
