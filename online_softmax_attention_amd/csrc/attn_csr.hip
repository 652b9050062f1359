// CSR segment softmax over given edge scores (gfx950): each destination row
// takes the softmax of its edges' scores and sums the gathered source value
// rows with those weights.
//
// Method: the relation view of the TIGA-lang attention pages -- a relation is
// a set of edges j -> i and each row's output is the softmax over its edges
// against the source values -- with the scores supplied as an edge field, the
// CSR case the varlen-by-graph-composition section names for compiled
// streaming.  No MFMA: the work is a gather, bound by memory.
//
// One wave per (row, head).  Workgroups go to the 8 XCDs round-robin; when H
// divides 8 or 8 divides H each XCD takes the rows of one head at a time, so
// its L2 holds that head's value rows (random gathers over a quarter of the
// values instead of all of them at H = 4); otherwise the head index varies
// fastest.  Pass 1: the row maximum over the segment's scores (64 edges per
// load).  Pass 2: the 64 lanes form 8 edge slots x 8 feature parts; a slot
// gathers kCsrUnroll source rows per step with 16-byte loads (a 128-
// or 256-byte row split over its 8 lanes), all issued before the first is
// used, weights them by exp(s - m) and accumulates in f32 in edge order; the
// slots then reduce across lanes.  The row pointer and
// column indices are clamped into range, so malformed CSR gives wrong results
// but no out-of-bounds access.
#include "attn_device.h"

namespace osattn {

// One-wave workgroups, five edges per slot per step: measured on the 65536-row
// graph (H=4, D=64 fp16) against four-wave workgroups with four edges per
// step, 184 -> 170 us (two waves 180 us; eight edges per step spill, 445 us).
constexpr int kCsrWaves = 1;
constexpr int kCsrUnroll = 5;  // edges per slot per step (row loads in flight per lane)

template <typename T, int D>
__global__ void __launch_bounds__(64 * kCsrWaves) csr_softmax_kernel(CsrParams p) {
    constexpr int esz = (int)sizeof(T);
    constexpr int CH = D * esz / 16;   // 16-byte chunks per value row
    constexpr int NCH = CH / 8;        // chunks per lane
    constexpr int EPC = 16 / esz;      // elements per chunk
    static_assert(NCH * 8 == CH, "a value row must split over 8 lanes");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int h, i;
    if (p.heads_by_xcd) {
        const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
        int rb;
        if (p.H <= 8) {  // 8 / H XCDs per head, row blocks dealt among them
            const int per = 8 / p.H;
            h = xcd % p.H;
            rb = j * per + xcd / p.H;
        } else {  // H / 8 heads per XCD, one after the other
            h = xcd + 8 * (j / p.row_blocks);
            rb = j % p.row_blocks;
        }
        if (rb >= p.row_blocks) return;
        i = rb * kCsrWaves + wave;
        if (i >= p.n_dst) return;
    } else {
        const int64_t r = (int64_t)blockIdx.x * kCsrWaves + wave;
        if (r >= (int64_t)p.H * p.n_dst) return;
        h = (int)(r % p.H);
        i = (int)(r / p.H);
    }
    const int nnz = p.nnz;
    int lo = p.row_ptr[i], hi = p.row_ptr[i + 1];
    lo = lo < 0 ? 0 : (lo > nnz ? nnz : lo);
    hi = hi < lo ? lo : (hi > nnz ? nnz : hi);
    const float *sh = p.scores + (int64_t)h * p.s_sh;

    // Pass 1: the row maximum.
    float mx = kNegInf;
    for (int e = lo + lane; e < hi; e += 64) mx = vmax(mx, sh[e]);
    mx = xor32_max(mx);
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) mx = vmax(mx, __shfl_xor(mx, off));

    // Pass 2: weights and the gathered, weighted value rows.
    const int slot = lane >> 3, part = lane & 7;
    const char *vh = static_cast<const char *>(p.v) + (int64_t)h * p.v_sh * esz;
    float acc[NCH][EPC];
#pragma unroll
    for (int k = 0; k < NCH; ++k)
#pragma unroll
        for (int t = 0; t < EPC; ++t) acc[k][t] = 0.f;
    float lsum = 0.f;
    const float m0 = (mx == kNegInf) ? 0.f : mx;  // a row of -inf scores weighs nothing
    // Each step takes kCsrUnroll edges per slot and issues all their gathers
    // before the first use, so every lane has that many row loads in flight.
    for (int e0 = lo + slot; e0 < hi; e0 += 8 * kCsrUnroll) {
        float w[kCsrUnroll];
        u32x4 raw[kCsrUnroll][NCH];
#pragma unroll
        for (int u = 0; u < kCsrUnroll; ++u) {
            const int e = e0 + 8 * u;
            const bool in = e < hi;
            const int es = in ? e : e0;  // an edge past the row's end re-reads e0 and weighs 0
            int col = p.col_idx[es];
            col = col < 0 ? 0 : (col >= p.n_src ? p.n_src - 1 : col);
            const char *vrow = vh + (int64_t)col * p.v_sn * esz;
#pragma unroll
            for (int k = 0; k < NCH; ++k) raw[u][k] = *reinterpret_cast<const u32x4 *>(vrow + (part + 8 * k) * 16);
            const float wu = fast_exp2((sh[es] - m0) * kLog2e);
            w[u] = in ? wu : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kCsrUnroll; ++u) {
            if (part == 0) lsum += w[u];
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                if constexpr (esz == 4) {
                    const f32x4 x = __builtin_bit_cast(f32x4, raw[u][k]);
#pragma unroll
                    for (int t = 0; t < 4; ++t) acc[k][t] = fmaf(w[u], x[t], acc[k][t]);
                } else {
                    typedef typename Half8<T>::vec vec8;
                    const vec8 x = __builtin_bit_cast(vec8, raw[u][k]);
#pragma unroll
                    for (int t = 0; t < 8; ++t) acc[k][t] = fmaf(w[u], (float)x[t], acc[k][t]);
                }
            }
        }
    }
    // Sum the 8 edge slots (lane bits 3..5) and the row's weight total.
#pragma unroll
    for (int k = 0; k < NCH; ++k)
#pragma unroll
        for (int t = 0; t < EPC; ++t) {
            float x = acc[k][t];
            x += __shfl_xor(x, 8);
            x += __shfl_xor(x, 16);
            x = xor32_sum(x);
            acc[k][t] = x;
        }
    lsum = xor32_sum(lsum);
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);

    if (slot == 0) {
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;  // an empty row stores zeros
        float *orow = p.o + (int64_t)h * p.o_sh + (int64_t)i * p.o_sn;
#pragma unroll
        for (int k = 0; k < NCH; ++k)
#pragma unroll
            for (int t = 0; t < EPC; t += 4) {
                f32x4 y = {acc[k][t] * inv, acc[k][t + 1] * inv, acc[k][t + 2] * inv, acc[k][t + 3] * inv};
                *reinterpret_cast<f32x4 *>(orow + (part + 8 * k) * EPC + t) = y;
            }
    }
    if (lane == 0) {
        p.m[(int64_t)h * p.n_dst + i] = mx;
        p.l[(int64_t)h * p.n_dst + i] = lsum;
    }
}

hipError_t launch_csr_softmax(int dtype, int d, CsrParams p, hipStream_t st) {
    const int64_t waves = (int64_t)p.H * p.n_dst;
    int64_t grid = (waves + kCsrWaves - 1) / kCsrWaves;
    const int64_t nb = ((int64_t)p.n_dst + kCsrWaves - 1) / kCsrWaves;
    p.row_blocks = (int)nb;
    p.heads_by_xcd = (8 % p.H == 0 || p.H % 8 == 0) ? 1 : 0;
    if (p.heads_by_xcd) {
        const int64_t per = p.H <= 8 ? 8 / p.H : 1;
        grid = p.H <= 8 ? 8 * ((nb + per - 1) / per) : (int64_t)p.H * nb;
    }
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 g((unsigned)grid), b(64 * kCsrWaves);
    if (dtype == 0) {
        if (d == 64) hipLaunchKernelGGL((csr_softmax_kernel<float, 64>), g, b, 0, st, p);
        else hipLaunchKernelGGL((csr_softmax_kernel<float, 128>), g, b, 0, st, p);
    } else if (dtype == 1) {
        if (d == 64) hipLaunchKernelGGL((csr_softmax_kernel<_Float16, 64>), g, b, 0, st, p);
        else hipLaunchKernelGGL((csr_softmax_kernel<_Float16, 128>), g, b, 0, st, p);
    } else {
        if (d == 64) hipLaunchKernelGGL((csr_softmax_kernel<__bf16, 64>), g, b, 0, st, p);
        else hipLaunchKernelGGL((csr_softmax_kernel<__bf16, 128>), g, b, 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace osattn
