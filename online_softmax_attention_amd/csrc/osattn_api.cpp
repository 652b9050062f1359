// C ABI of the attention library: host-side argument checks, the backward's
// workspace plan, and dispatch to the HIP kernels.  Declared in osattn.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "../../include/osattn.h"
#include "api_internal.h"
#include "attn_params.h"

namespace osattn {
hipError_t launch_forward(int dtype, int d, int mask, FwdParams p, int max_seqlen, hipStream_t st);
hipError_t launch_backward(int d, int mask, BwdParams p, int seqs, hipStream_t st);
hipError_t launch_backward16(int dtype, int d, int mask, BwdParams p, int seqs, int sched_shift,
                             hipStream_t st);
hipError_t launch_forward_pruned(int dtype, int d, FwdParams p, hipStream_t st);
int fwd16_block_keys(int d, int waves);
hipError_t launch_csr_softmax(int dtype, int d, CsrParams p, hipStream_t st);
}  // namespace osattn

using namespace osattn;

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_err[0] = '\0';
    return OSATTN_OK;
}

size_t elem_size(int dtype) { return dtype == OSATTN_F32 ? 4 : 2; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxLen = (int64_t)1 << 30;
constexpr int64_t kMaxRowBytes = (int64_t)1 << 22;  // 4 MiB between consecutive rows

// Checks shared by the forward and the backward.  Returns OSATTN_OK or an
// error status with g_err set.
int check_common(int dtype, int H, int64_t n_q, int64_t n_k, int d, float scale, int causal,
                 const int32_t *cu, int num_seqs, int max_seqlen) {
    if (dtype != OSATTN_F32 && dtype != OSATTN_F16 && dtype != OSATTN_BF16)
        return fail(OSATTN_ERR_INVALID_ARG, "dtype %d is not OSATTN_F32/F16/BF16", dtype);
    if (H <= 0) return fail(OSATTN_ERR_INVALID_ARG, "H must be positive (got %d)", H);
    if (n_q <= 0 || n_k <= 0)
        return fail(OSATTN_ERR_INVALID_ARG, "n_q and n_k must be positive (got %lld, %lld)",
                    (long long)n_q, (long long)n_k);
    if (n_q > kMaxLen || n_k > kMaxLen)
        return fail(OSATTN_ERR_UNSUPPORTED, "n_q and n_k must be <= 2^30");
    if (d <= 0) return fail(OSATTN_ERR_INVALID_ARG, "d must be positive (got %d)", d);
    if (!std::isfinite(scale)) return fail(OSATTN_ERR_UNSUPPORTED, "scale must be finite");
    if (!(scale > 0.f)) return fail(OSATTN_ERR_UNSUPPORTED, "scale must be > 0");
    if (cu) {
        if (num_seqs <= 0) return fail(OSATTN_ERR_INVALID_ARG, "num_seqs must be positive with cu_seqlens");
        if (n_q != n_k) return fail(OSATTN_ERR_INVALID_ARG, "varlen needs n_q == n_k (total tokens)");
        if (max_seqlen <= 0 || max_seqlen > n_q)
            return fail(OSATTN_ERR_INVALID_ARG, "max_seqlen must be in [1, n_q] (got %d)", max_seqlen);
    } else if (causal && n_q != n_k) {
        return fail(OSATTN_ERR_INVALID_ARG, "causal attention needs n_q == n_k (got %lld, %lld)",
                    (long long)n_q, (long long)n_k);
    }
    return OSATTN_OK;
}

// O's element type: f32 for any input, or the 16-bit input type itself.
int check_o_dtype(int dtype, int o_dtype, size_t *es_o) {
    if (o_dtype == OSATTN_F32) {
        *es_o = 4;
        return 0;
    }
    if (dtype != OSATTN_F32 && o_dtype == dtype) {
        *es_o = 2;
        return 0;
    }
    return fail(OSATTN_ERR_INVALID_ARG, "o_dtype must be OSATTN_F32 or the input dtype (got %d for %d)",
                o_dtype, dtype);
}

int check_tensor(const char *name, const void *p, int64_t sh, int64_t sn, size_t esize) {
    if (!p) return fail(OSATTN_ERR_INVALID_ARG, "%s is NULL", name);
    if (sh < 0 || sn < 0) return fail(OSATTN_ERR_INVALID_ARG, "%s has a negative stride", name);
    if (!aligned16(p)) return fail(OSATTN_ERR_ALIGNMENT, "%s is not 16-byte aligned", name);
    const int64_t q = 16 / (int64_t)esize;
    if (sh % q || sn % q)
        return fail(OSATTN_ERR_ALIGNMENT, "%s strides (%lld, %lld) are not multiples of %lld elements",
                    name, (long long)sh, (long long)sn, (long long)q);
    return OSATTN_OK;
}

// Compute units of the current device (cached per device; 256 if unknown).
// Threads may race to fill an entry; they store the same value.
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// ---------------------------------------------------------------- fwd plan
// Split-KV applies to the 16-bit dense forward when its query tiles cannot
// occupy half the device AND each would scan many key blocks alone (long keys,
// few queries: decode-like shapes), and to the f32 dense forward whenever its
// tiles cannot fill the device's workgroup slots and the keys span at least
// four 128-key units.  The key range is cut into 128-key-aligned pieces.  A split costs a second (combine) launch of a few microseconds, which
// is why short key ranges are not split: measured on MI355X, N=1024 H=4 D=64
// ran 15 us unsplit vs 9 + 8 us split.
struct FwdPlan {
    int n_tiles, splits, split_len;
    int tile_rows;               // query rows per 16-bit tile
    int pair;                    // causal: two tiles (T-1-i, i) per workgroup
    int waves;                   // waves per 128-row-tile workgroup (8, or 4: two per CU)
    int sched_max, sched_shift;  // varlen work list (0: none)
    int sched_inline;            // varlen, <= 64 sequences: items ranked in-kernel, no list
    int f32_groups;              // f32 dense d = 64: 4 = 32-row tiles of four key groups, else 1
    size_t total;                // workspace bytes (0: none used)
};

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Varlen work-list plan shared by the forward and the backward: false when no
// list is used.  n == S * max_seqlen means every sequence has max_seqlen tokens:
// the natural grid is then balanced already and the list would only add a
// launch.
bool plan_varlen_sched(int H, int64_t n_q, int bc, int num_seqs, int max_seqlen, int *sched_max,
                       int *sched_shift) {
    if (num_seqs <= 0 || max_seqlen <= 0 || n_q == (int64_t)num_seqs * max_seqlen) return false;
    const int64_t S = num_seqs, t_max = (max_seqlen + 127) / 128;
    int64_t tiles = (n_q + 127 * S) / 128;
    if (S * t_max < tiles) tiles = S * t_max;
    int64_t bound = (tiles + S) / 2;
    if (S * ((t_max + 1) / 2) < bound) bound = S * ((t_max + 1) / 2);
    if (bound <= 0 || bound * H > 0x7fffffffLL) return false;
    const int64_t max_w = 2 * ((max_seqlen + bc - 1) / bc);
    int shift = 0;
    while ((max_w >> shift) >= kSchedBins) ++shift;
    *sched_max = (int)bound;
    *sched_shift = shift;
    return true;
}

// Varlen (16-bit): a schedule kernel sorts the varlen items (tile pairs
// (T-1-i, i) of one sequence) by the key blocks they scan, largest first, into
// the workspace, and the forward takes its items from that list (without a
// workspace it walks the natural (sequence, pair) grid instead).  A sequence of
// T_s tiles has ceil(T_s / 2) items, so the list holds at most
// (sum_s T_s + S) / 2 entries, with sum_s T_s <= (n + 127 S) / 128 and
// T_s <= ceil(max_seqlen / 128).
FwdPlan plan_forward(int dtype, int H, int64_t n_q, int64_t n_k, int d, int causal,
                     const int32_t *cu, int num_seqs, int max_seqlen) {
    FwdPlan pl{};
    pl.n_tiles = (int)((n_q + 127) / 128);
    pl.splits = 1;
    pl.split_len = (int)n_k;
    if (dtype != OSATTN_F32 && !causal && !cu) {
        const int64_t items = (int64_t)H * pl.n_tiles;
        const int64_t target = device_cus();
        const int64_t blocks = (n_k + (d == 64 ? 255 : 127)) / (d == 64 ? 256 : 128);
        if (2 * items <= target && blocks >= 16) {
            const int64_t units = (n_k + 127) / 128;
            int64_t splits = (target + items - 1) / items;
            if (splits > units) splits = units;
            if (splits > 64) splits = 64;
            const int64_t per = (units + splits - 1) / splits;
            pl.splits = (int)((units + per - 1) / per);
            pl.split_len = (int)(per * 128);
        }
    } else if (dtype == OSATTN_F32 && !causal && !cu) {
        // f32: 128-row tiles of 4 waves; split the keys until there is about one
        // workgroup per CU.  Measured on MI355X (SQ=8192 SK=2048 H=1 D=64): 149 us
        // unsplit (64 workgroups), 52 us in 4 splits, 55 us in 8 (two per CU).
        // At d = 64, keys too few to split (under 512) take 32-row tiles whose
        // four waves share every key block instead: four times the workgroups
        // (N=128 H=1: 12.6 -> 6.6 us).  So do problems whose 32-row tiles alone
        // give every CU a workgroup: no partial states are written and read
        // back, for a little time (SQ=8192 SK=2048 H=1: 50.5 us against 48.9 us
        // split, 8.9 MB of partials gone).  Smaller grids split the keys
        // (N=1024 H=4: 23.2 us split vs 26.7 us in 32-row tiles).
        const int64_t items = (int64_t)H * pl.n_tiles;
        const int64_t target = device_cus();
        const int64_t units = (n_k + 127) / 128;
        const int64_t items32 = (int64_t)H * ((n_q + 31) / 32);
        if (d == 64 && items < target && (units < 4 || items32 >= target)) {
            pl.f32_groups = 4;
        } else if (items < target && units >= 4) {
            int64_t splits = (target + items - 1) / items;
            if (splits > units) splits = units;
            if (splits > 64) splits = 64;
            const int64_t per = (units + splits - 1) / splits;
            pl.splits = (int)((units + per - 1) / per);
            pl.split_len = (int)(per * 128);
        }
    }
    if (pl.splits > 1) pl.total = round256((size_t)pl.splits * H * n_q * (d + 4) * sizeof(float));
    // Dense / causal problems whose 128-row tiles (pairs, causal) would not
    // give every CU a workgroup use 64- or 32-row tiles: the workgroup's 8
    // waves then split each key block 4 or 8 ways instead of 2, so more
    // workgroups each scan the keys with more waves per row.  Measured on
    // MI355X against stopping at half the CUs: causal N=2048 H=16 D=128
    // 42.3 -> 34.6 us, causal N=4096 H=8 D=64 47.8 -> 33.3 us; dense shapes at
    // that boundary ran the same either way.
    // Causal tiles are paired (T-1-i, i) so that every workgroup does equal
    // work, unless the 128-row tiles alone cannot fill the device: then each
    // workgroup takes one tile, heaviest first, to keep the serial chain short.
    pl.tile_rows = 128;
    pl.pair = causal && (int64_t)H * ((n_q + 127) / 128) >= device_cus();
    if (dtype != OSATTN_F32 && !cu && pl.splits == 1) {
        const int64_t cus = device_cus();
        const auto items = [&](int64_t tr) {
            const int64_t t = (n_q + tr - 1) / tr;
            return (int64_t)H * (pl.pair ? (t + 1) / 2 : t);
        };
        while (pl.tile_rows > (d == 64 ? 32 : 64) && items(pl.tile_rows) < cus) pl.tile_rows /= 2;
    }
    // Dense and causal 128-row tiles run on the 8-wave pipelined kernel; the
    // tiled kernel (fwd16) keeps the 64- and 32-row tiles with 8 waves and the
    // varlen tiles of short sequences with four-wave workgroups (64 KiB of
    // LDS, two per CU, blocks of half as many keys: varlen causal 16k tokens
    // H=8 D=64 62 -> 49 us against 8 waves).
    pl.waves = (dtype != OSATTN_F32 && cu) ? 4 : 8;
    // Varlen order: up to 64 sequences, each workgroup ranks its own tile pair
    // (sequences by tile count, no extra launch: 16k tokens in 20 sequences,
    // H=8 D=64: 47.4 + 4.9 us with the list kernel); more sequences use the
    // list kernel's counting sort, written to the workspace.
    if (dtype != OSATTN_F32 && cu && plan_varlen_sched(H, n_q, fwd16_block_keys(d, pl.waves),
                                                       num_seqs, max_seqlen, &pl.sched_max,
                                                       &pl.sched_shift)) {
        if (num_seqs <= 64) pl.sched_inline = 1;
        else pl.total = round256(16 + 16 * (size_t)pl.sched_max);
    }
    return pl;
}

int mask_kind(int causal, const int32_t *cu) {
    if (cu) return causal ? kVarlenCausal : kVarlen;
    return causal ? kCausal : kDense;
}

// ---------------------------------------------------------------- bwd plan
struct BwdPlan {
    int q_tiles, k_tiles, q_splits, k_splits, seqs;
    int pair_k, pair_q;          // fp16/bf16 causal: items of two tiles (i, T-1-i)
    int sched_max, sched_shift;  // fp16/bf16 varlen work list (0: none)
    size_t off_delta, off_mlog2, off_linv, off_dq, off_dk, off_dv, off_sched, total;
};

int clampi(int64_t x, int lo, int hi) { return (int)(x < lo ? lo : (x > hi ? hi : x)); }

BwdPlan plan_backward(int dtype, int H, int64_t n_q, int64_t n_k, int d, int causal, const int32_t *cu,
                      int num_seqs, int max_seqlen) {
    BwdPlan pl{};
    const bool varlen = cu != nullptr;
    pl.seqs = varlen ? num_seqs : 1;
    const int64_t qlen = varlen ? max_seqlen : n_q;
    const int64_t klen = varlen ? max_seqlen : n_k;
    pl.q_tiles = (int)((qlen + 127) / 128);
    pl.k_tiles = (int)((klen + 127) / 128);
    // Workgroups per pass to aim for; a split keeps at least 256 positions of
    // the reduced axis.  Every backward kernel runs one workgroup per CU, so a
    // second round of workgroups only adds partial sums to write and reduce.
    // f32: one round per pass (SQ=8192 SK=2048 H=1 D=64: 162.4 -> 155.1 us
    // against two rounds).  fp16/bf16 runs both passes in one launch: dense aims
    // at half the CUs per pass, one round in all (N=4096 H=1 D=128 bf16: 81.3
    // -> 52.6 us; N=2048 H=2 D=64 fp16: 36.7 -> 29.8 us); causal items are
    // unequal and balance better with a full round per pass (N=4096 H=2 D=128:
    // 82.1 -> 65.0 us, 72.8 us at half).
    const int64_t cus = device_cus();
    const int64_t target = (dtype == OSATTN_F32 || causal) ? cus : cus / 2;
    const int64_t base_k = (int64_t)H * pl.seqs * pl.k_tiles;
    const int64_t base_q = (int64_t)H * pl.seqs * pl.q_tiles;
    pl.k_splits = varlen ? 1 : clampi((target + base_k - 1) / base_k, 1, clampi(n_q / 256, 1, 16));
    pl.q_splits = varlen ? 1 : clampi((target + base_q - 1) / base_q, 1, clampi(n_k / 256, 1, 16));
    pl.pair_k = dtype != OSATTN_F32 && causal && !varlen && pl.k_splits == 1;
    pl.pair_q = dtype != OSATTN_F32 && causal && !varlen && pl.q_splits == 1;
    size_t off = 0;
    const size_t rowbytes = round256((size_t)H * n_q * sizeof(float));
    pl.off_delta = off; off += rowbytes;
    pl.off_mlog2 = off; off += rowbytes;
    pl.off_linv = off;  off += rowbytes;
    pl.off_dq = off;
    if (pl.q_splits > 1) off += round256((size_t)pl.q_splits * H * n_q * d * sizeof(float));
    pl.off_dk = off;
    if (pl.k_splits > 1) off += round256((size_t)pl.k_splits * H * n_k * d * sizeof(float));
    pl.off_dv = off;
    if (pl.k_splits > 1) off += round256((size_t)pl.k_splits * H * n_k * d * sizeof(float));
    pl.off_sched = off;
    if (dtype != OSATTN_F32 && varlen &&
        plan_varlen_sched(H, n_q, fwd16_block_keys(d, 8), num_seqs, max_seqlen, &pl.sched_max,
                          &pl.sched_shift))
        off += round256(16 + 16 * (size_t)pl.sched_max);
    pl.total = off;
    return pl;
}

int check_bwd_supported(int d) {
    if (d != 64 && d != 128)
        return fail(OSATTN_ERR_UNSUPPORTED, "backward supports d = 64 or 128 (got %d)", d);
    return OSATTN_OK;
}

}  // namespace

namespace osattn {

int set_error(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

// Every host check of osattn_bwd that does not involve the workspace.
int bwd_check_args(int dtype, int o_dtype, int H, int64_t n_q, int64_t n_k, int d, const void *q,
                   const void *k, const void *v, const void *o, const void *d_o,
                   int64_t q_stride_h, int64_t q_stride_n, int64_t kv_stride_h,
                   int64_t kv_stride_n, int64_t o_stride_h, int64_t o_stride_n, const float *m,
                   const float *l, float scale, int causal, const int32_t *cu_seqlens,
                   int num_seqs, int max_seqlen, void *dq, void *dk, void *dv) {
    int st = check_common(dtype, H, n_q, n_k, d, scale, causal, cu_seqlens, num_seqs, max_seqlen);
    if (st) return st;
    if ((st = check_bwd_supported(d))) return st;
    size_t es_o = 4;
    if ((st = check_o_dtype(dtype, o_dtype, &es_o))) return st;
    const size_t es = elem_size(dtype);
    if ((st = check_tensor("q", q, q_stride_h, q_stride_n, es))) return st;
    if ((st = check_tensor("k", k, kv_stride_h, kv_stride_n, es))) return st;
    if ((st = check_tensor("v", v, kv_stride_h, kv_stride_n, es))) return st;
    if ((st = check_tensor("d_o", d_o, q_stride_h, q_stride_n, es))) return st;
    if ((st = check_tensor("o", o, o_stride_h, o_stride_n, es_o))) return st;
    if ((st = check_tensor("dq", dq, q_stride_h, q_stride_n, es))) return st;
    if ((st = check_tensor("dk", dk, kv_stride_h, kv_stride_n, es))) return st;
    if ((st = check_tensor("dv", dv, kv_stride_h, kv_stride_n, es))) return st;
    // The backward kernels form offsets within a block of rows in 32 bits, as
    // the forward's do.
    if (q_stride_n * (int64_t)es > kMaxRowBytes || kv_stride_n * (int64_t)es > kMaxRowBytes)
        return fail(OSATTN_ERR_UNSUPPORTED, "row strides above %lld bytes are not supported",
                    (long long)kMaxRowBytes);
    if (!m || !l) return fail(OSATTN_ERR_INVALID_ARG, "m and l must not be NULL");
    return OSATTN_OK;
}

}  // namespace osattn

namespace {

// Launches the backward of checked arguments with the planned workspace.
int bwd_launch(int dtype, size_t es_o, int H, int64_t n_q, int64_t n_k, int d, const void *q,
               const void *k, const void *v, const void *o, const void *d_o, int64_t q_stride_h,
               int64_t q_stride_n, int64_t kv_stride_h, int64_t kv_stride_n, int64_t o_stride_h,
               int64_t o_stride_n, const float *m, const float *l, float scale, int causal,
               const int32_t *cu_seqlens, int num_seqs, void *dq, void *dk, void *dv,
               const BwdPlan &pl, char *ws, hipStream_t hs) {
    BwdParams p{};
    p.q = q; p.k = k; p.v = v; p.d_o = d_o;
    p.o = o; p.m = m; p.l = l;
    p.o16 = es_o == 2;
    p.dq = dq; p.dk = dk; p.dv = dv;
    p.q_sh = q_stride_h; p.q_sn = q_stride_n;
    p.kv_sh = kv_stride_h; p.kv_sn = kv_stride_n;
    p.o_sh = o_stride_h; p.o_sn = o_stride_n;
    p.H = H; p.n_q = (int)n_q; p.n_k = (int)n_k;
    p.num_seqs = cu_seqlens ? num_seqs : 1;
    p.cu = cu_seqlens;
    p.scale = scale;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.stat_delta = reinterpret_cast<float *>(ws + pl.off_delta);
    p.stat_mlog2 = reinterpret_cast<float *>(ws + pl.off_mlog2);
    p.stat_linv = reinterpret_cast<float *>(ws + pl.off_linv);
    p.dq_part = reinterpret_cast<float *>(ws + pl.off_dq);
    p.dk_part = reinterpret_cast<float *>(ws + pl.off_dk);
    p.dv_part = reinterpret_cast<float *>(ws + pl.off_dv);
    p.q_tiles = pl.q_tiles; p.k_tiles = pl.k_tiles;
    p.q_splits = pl.q_splits; p.k_splits = pl.k_splits;
    p.pair_k = pl.pair_k; p.pair_q = pl.pair_q;
    if (pl.sched_max > 0) {
        p.sched = reinterpret_cast<int32_t *>(ws + pl.off_sched);
        p.sched_max = pl.sched_max;
    }
    const int mk = mask_kind(causal, cu_seqlens);
    const hipError_t e = dtype == OSATTN_F32 ? launch_backward(d, mk, p, pl.seqs, hs)
                                             : launch_backward16(dtype, d, mk, p, pl.seqs,
                                                                 pl.sched_shift, hs);
    if (e != hipSuccess) return fail(OSATTN_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int osattn_version(void) { return 100; }

const char *osattn_status_string(int status) {
    switch (status) {
        case OSATTN_OK: return "OSATTN_OK";
        case OSATTN_ERR_INVALID_ARG: return "OSATTN_ERR_INVALID_ARG: invalid argument";
        case OSATTN_ERR_UNSUPPORTED: return "OSATTN_ERR_UNSUPPORTED: unsupported combination";
        case OSATTN_ERR_ALIGNMENT: return "OSATTN_ERR_ALIGNMENT: pointer or stride not 16-byte aligned";
        case OSATTN_ERR_HIP: return "OSATTN_ERR_HIP: HIP runtime error";
        case OSATTN_ERR_WORKSPACE: return "OSATTN_ERR_WORKSPACE: workspace missing or too small";
        default: return "unknown osattn status";
    }
}

const char *osattn_last_error_message(void) { return g_err; }

size_t osattn_fwd_workspace_bytes(int dtype, int H, int64_t n_q, int64_t n_k, int d, int causal,
                                  const int32_t *cu_seqlens, int num_seqs, int max_seqlen) {
    if (check_common(dtype, H, n_q, n_k, d, 1.f, causal, cu_seqlens, num_seqs, max_seqlen)) return 0;
    if (d != 64 && d != 128) return 0;
    return plan_forward(dtype, H, n_q, n_k, d, causal, cu_seqlens, num_seqs, max_seqlen).total;
}

int osattn_fwd(int dtype, int o_dtype, int H, int64_t n_q, int64_t n_k, int d, const void *q,
               const void *k, const void *v, int64_t q_stride_h, int64_t q_stride_n,
               int64_t kv_stride_h, int64_t kv_stride_n, void *o, int64_t o_stride_h,
               int64_t o_stride_n, float *m, float *l, float scale, int causal,
               const int32_t *cu_seqlens, int num_seqs, int max_seqlen, void *workspace,
               size_t workspace_bytes, void *stream) {
    int st = check_common(dtype, H, n_q, n_k, d, scale, causal, cu_seqlens, num_seqs, max_seqlen);
    if (st) return st;
    if (d != 64 && d != 128)
        return fail(OSATTN_ERR_UNSUPPORTED, "forward supports d = 64 or 128 (got %d)", d);
    size_t es_o = 4;
    if ((st = check_o_dtype(dtype, o_dtype, &es_o))) return st;
    const size_t es = elem_size(dtype);
    if ((st = check_tensor("q", q, q_stride_h, q_stride_n, es))) return st;
    if ((st = check_tensor("k", k, kv_stride_h, kv_stride_n, es))) return st;
    if ((st = check_tensor("v", v, kv_stride_h, kv_stride_n, es))) return st;
    if ((st = check_tensor("o", o, o_stride_h, o_stride_n, es_o))) return st;
    // The kernels address one 256-row block with 32-bit byte offsets.
    if (q_stride_n * (int64_t)es > kMaxRowBytes || kv_stride_n * (int64_t)es > kMaxRowBytes)
        return fail(OSATTN_ERR_UNSUPPORTED, "row strides above %lld bytes are not supported",
                    (long long)kMaxRowBytes);
    if (!m || !l) return fail(OSATTN_ERR_INVALID_ARG, "m and l must not be NULL");

    FwdParams p{};
    p.q = q; p.k = k; p.v = v;
    p.o = o; p.m = m; p.l = l;
    p.o16 = es_o == 2;
    p.q_sh = q_stride_h; p.q_sn = q_stride_n;
    p.kv_sh = kv_stride_h; p.kv_sn = kv_stride_n;
    p.o_sh = o_stride_h; p.o_sn = o_stride_n;
    p.H = H; p.n_q = (int)n_q; p.n_k = (int)n_k;
    p.num_seqs = cu_seqlens ? num_seqs : 1;
    p.cu = cu_seqlens;
    p.scale = scale;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.splits = 1;
    p.split_len = (int)n_k;
    p.tile_rows = 128;
    p.pair = 1;
    const FwdPlan pl = plan_forward(dtype, H, n_q, n_k, d, causal, cu_seqlens, num_seqs, max_seqlen);
    if (pl.total > 0 && workspace && workspace_bytes >= pl.total) {
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(OSATTN_ERR_ALIGNMENT, "workspace is not 256-byte aligned");
        if (pl.splits > 1) {
            p.part = static_cast<float *>(workspace);
            p.splits = pl.splits;
            p.split_len = pl.split_len;
        }
        if (pl.sched_max > 0 && !pl.sched_inline) {
            p.sched = static_cast<int32_t *>(workspace);
            p.sched_max = pl.sched_max;
            p.sched_shift = pl.sched_shift;
        }
    }
    if (pl.sched_inline) {
        p.sched_inline = 1;
        p.sched_max = pl.sched_max;
    }
    if (p.splits == 1) p.tile_rows = pl.tile_rows;
    p.pair = pl.pair;
    p.waves = pl.waves;
    p.f32_groups = pl.f32_groups == 4 ? 4 : 1;
    const hipError_t e = launch_forward(dtype, d, mask_kind(causal, cu_seqlens), p, max_seqlen,
                                        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(OSATTN_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
    return ok();
}

int osattn_fwd_pruned(int dtype, int o_dtype, int H, int64_t n_q, int64_t n_k, int d,
                      const void *q, const void *k, const void *v, int64_t q_stride_h,
                      int64_t q_stride_n, int64_t kv_stride_h, int64_t kv_stride_n, void *o,
                      int64_t o_stride_h, int64_t o_stride_n, float *m, float *l, float scale,
                      float rho, void *stream) {
    int st = check_common(dtype, H, n_q, n_k, d, scale, 0, nullptr, 0, 0);
    if (st) return st;
    if (dtype == OSATTN_F32)
        return fail(OSATTN_ERR_UNSUPPORTED, "tile pruning supports fp16/bf16 only");
    if (d != 64 && d != 128) return fail(OSATTN_ERR_UNSUPPORTED, "d must be 64 or 128 (got %d)", d);
    if (!(rho > 0.f && rho <= 1.f))
        return fail(OSATTN_ERR_INVALID_ARG, "rho must be in (0, 1] (got %g); omit pruning for the "
                    "exact result", (double)rho);
    size_t es_o = 4;
    if ((st = check_o_dtype(dtype, o_dtype, &es_o))) return st;
    const size_t es = elem_size(dtype);
    if ((st = check_tensor("q", q, q_stride_h, q_stride_n, es))) return st;
    if ((st = check_tensor("k", k, kv_stride_h, kv_stride_n, es))) return st;
    if ((st = check_tensor("v", v, kv_stride_h, kv_stride_n, es))) return st;
    if ((st = check_tensor("o", o, o_stride_h, o_stride_n, es_o))) return st;
    if (q_stride_n * (int64_t)es > kMaxRowBytes || kv_stride_n * (int64_t)es > kMaxRowBytes)
        return fail(OSATTN_ERR_UNSUPPORTED, "row strides above %lld bytes are not supported",
                    (long long)kMaxRowBytes);
    if (!m || !l) return fail(OSATTN_ERR_INVALID_ARG, "m and l must not be NULL");
    FwdParams p{};
    p.q = q; p.k = k; p.v = v;
    p.o = o; p.m = m; p.l = l;
    p.o16 = es_o == 2;
    p.q_sh = q_stride_h; p.q_sn = q_stride_n;
    p.kv_sh = kv_stride_h; p.kv_sn = kv_stride_n;
    p.o_sh = o_stride_h; p.o_sn = o_stride_n;
    p.H = H; p.n_q = (int)n_q; p.n_k = (int)n_k;
    p.num_seqs = 1;
    p.scale = scale;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.splits = 1;
    p.split_len = (int)n_k;
    p.tile_rows = 128;
    p.pair = 0;
    p.prune_thr = logf(rho) / scale;
    const hipError_t e = launch_forward_pruned(dtype, d, p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(OSATTN_ERR_HIP, "pruned forward launch: %s", hipGetErrorString(e));
    return ok();
}

int osattn_csr_softmax(int dtype, int H, int64_t n_dst, int64_t n_src, int d,
                       const int32_t *row_ptr, const int32_t *col_idx, int64_t nnz,
                       const float *scores, int64_t scores_stride_h, const void *v,
                       int64_t v_stride_h, int64_t v_stride_n, float *o, int64_t o_stride_h,
                       int64_t o_stride_n, float *m, float *l, void *stream) {
    if (dtype != OSATTN_F32 && dtype != OSATTN_F16 && dtype != OSATTN_BF16)
        return fail(OSATTN_ERR_INVALID_ARG, "dtype %d is not OSATTN_F32/F16/BF16", dtype);
    if (H <= 0 || n_dst <= 0 || n_src <= 0 || nnz < 0)
        return fail(OSATTN_ERR_INVALID_ARG, "H, n_dst, n_src must be positive and nnz >= 0");
    if (n_dst > kMaxLen || n_src > kMaxLen || nnz > 0x7fffffffLL)
        return fail(OSATTN_ERR_UNSUPPORTED, "n_dst, n_src must be <= 2^30 and nnz < 2^31");
    if (d != 64 && d != 128) return fail(OSATTN_ERR_UNSUPPORTED, "d must be 64 or 128 (got %d)", d);
    if (!row_ptr) return fail(OSATTN_ERR_INVALID_ARG, "row_ptr is NULL");
    if (nnz > 0 && (!col_idx || !scores))
        return fail(OSATTN_ERR_INVALID_ARG, "col_idx and scores must not be NULL when nnz > 0");
    if (scores_stride_h < 0) return fail(OSATTN_ERR_INVALID_ARG, "scores_stride_h is negative");
    int st;
    const size_t es = elem_size(dtype);
    if ((st = check_tensor("v", v, v_stride_h, v_stride_n, es))) return st;
    if ((st = check_tensor("o", o, o_stride_h, o_stride_n, 4))) return st;
    if (!m || !l) return fail(OSATTN_ERR_INVALID_ARG, "m and l must not be NULL");
    CsrParams p{};
    p.row_ptr = row_ptr; p.col_idx = col_idx;
    p.scores = scores; p.s_sh = scores_stride_h;
    p.v = v; p.v_sh = v_stride_h; p.v_sn = v_stride_n;
    p.o = o; p.o_sh = o_stride_h; p.o_sn = o_stride_n;
    p.m = m; p.l = l;
    p.H = H; p.n_dst = (int)n_dst; p.n_src = (int)n_src; p.nnz = (int)nnz;
    const hipError_t e = launch_csr_softmax(dtype, d, p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(OSATTN_ERR_HIP, "csr softmax launch: %s", hipGetErrorString(e));
    return ok();
}

size_t osattn_bwd_workspace_bytes(int dtype, int H, int64_t n_q, int64_t n_k, int d, int causal,
                                  const int32_t *cu_seqlens, int num_seqs, int max_seqlen) {
    if (check_common(dtype, H, n_q, n_k, d, 1.f, causal, cu_seqlens, num_seqs, max_seqlen)) return 0;
    if (check_bwd_supported(d)) return 0;
    return plan_backward(dtype, H, n_q, n_k, d, causal, cu_seqlens, num_seqs, max_seqlen).total;
}

int osattn_bwd(int dtype, int o_dtype, int H, int64_t n_q, int64_t n_k, int d, const void *q,
               const void *k, const void *v, const void *o, const void *d_o, int64_t q_stride_h,
               int64_t q_stride_n, int64_t kv_stride_h, int64_t kv_stride_n, int64_t o_stride_h,
               int64_t o_stride_n, const float *m, const float *l, float scale, int causal,
               const int32_t *cu_seqlens, int num_seqs, int max_seqlen, void *dq, void *dk, void *dv,
               void *workspace, size_t workspace_bytes, void *stream) {
    int st = osattn::bwd_check_args(dtype, o_dtype, H, n_q, n_k, d, q, k, v, o, d_o, q_stride_h,
                                    q_stride_n, kv_stride_h, kv_stride_n, o_stride_h, o_stride_n,
                                    m, l, scale, causal, cu_seqlens, num_seqs, max_seqlen, dq, dk,
                                    dv);
    if (st) return st;
    size_t es_o = 4;
    check_o_dtype(dtype, o_dtype, &es_o);
    const BwdPlan pl = plan_backward(dtype, H, n_q, n_k, d, causal, cu_seqlens, num_seqs, max_seqlen);
    if (!workspace) return fail(OSATTN_ERR_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(OSATTN_ERR_ALIGNMENT, "workspace is not 256-byte aligned");
    if (workspace_bytes < pl.total)
        return fail(OSATTN_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, pl.total);
    return bwd_launch(dtype, es_o, H, n_q, n_k, d, q, k, v, o, d_o, q_stride_h, q_stride_n,
                      kv_stride_h, kv_stride_n, o_stride_h, o_stride_n, m, l, scale, causal,
                      cu_seqlens, num_seqs, dq, dk, dv, pl, static_cast<char *>(workspace),
                      static_cast<hipStream_t>(stream));
}

}  // extern "C"

