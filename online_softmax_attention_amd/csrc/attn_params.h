// Launch parameter blocks shared by the host dispatch code and the kernels.
#pragma once

#include <stdint.h>

namespace osattn {

// Mask kinds.  The relation decides which keys a query row admits.
enum MaskKind : int {
    kDense = 0,        // every key
    kCausal = 1,       // keys j <= i
    kVarlen = 2,       // keys of the row's own packed sequence
    kVarlenCausal = 3  // both
};

// Bins of the varlen work-list sort (sort keys are coarsened to fit).
constexpr int kSchedBins = 4096;

struct FwdParams {
    const void *q, *k, *v;
    void *o;               // f32, or the input dtype when o16 (16-bit inputs only)
    float *m, *l;
    int64_t q_sh, q_sn;    // element strides of q
    int64_t kv_sh, kv_sn;  // element strides of k and v
    int64_t o_sh, o_sn;    // element strides of o
    int H;
    int n_q, n_k;
    int n_tiles;           // query tiles per (head, sequence)
    int tile_rows;         // query rows per tile of the 16-bit kernel: 128, 64 or 32
    int pair;              // causal 16-bit: tile pairs (T-1-i, i) per workgroup (else one tile)
    int waves;             // 16-bit 128-row tiles: 8 waves per workgroup, or 4 (two per CU)
    int num_seqs;          // 1 unless varlen
    const int32_t *cu;     // device cumulative lengths (varlen) or null
    float scale;           // softmax scale
    float scale_log2;      // scale * log2(e)
    // Split-KV (dense relation only): the key range is cut into `splits`
    // pieces of `split_len` keys, one workgroup each; partial states go to
    // `part` ((splits, H, n_q, D + 4) f32: U then m_ref, m_max, l) and a second
    // launch combines them.  splits == 1: direct output.
    float *part;
    int splits, split_len;
    // Varlen work list (16-bit kernels).  When non-null, a schedule kernel
    // first writes sched[0] = number of items and, from sched + 4, sched_max
    // int4 entries {seq_lo, seq_hi, tile0, tile1} (tile1 = -1: one tile;
    // tile0 = -1: empty slot), ordered by the number of key blocks the item
    // scans, largest first.  The grid has sched_max * H workgroups;
    // sched_shift coarsens the sort key to fit the histogram.
    int32_t *sched;
    int sched_max, sched_shift;
    // Varlen with at most 64 sequences and no list: each workgroup finds its
    // own item (rank = blockIdx / H) among the tile pairs, sequences ordered by
    // tile count, most first; the grid has sched_max * H workgroups.
    int sched_inline;
    int o16;               // o holds the input dtype instead of f32
    float prune_thr;       // tile pruning: ln(rho) / scale (raw score units)
    int f32_groups;        // f32 dense, d = 64: 4 = 32-row tiles of four key groups, else 1
};

struct BwdParams {
    const void *q, *k, *v, *d_o;
    const void *o;         // the forward's output: f32, or the input dtype when o16
    const float *m, *l;
    int o16;
    void *dq, *dk, *dv;
    int64_t q_sh, q_sn;
    int64_t kv_sh, kv_sn;
    int64_t o_sh, o_sn;
    int H;
    int n_q, n_k;
    int num_seqs;
    const int32_t *cu;
    float scale, scale_log2;
    // workspace views
    float *stat_delta;     // (H, n_q): D_i = <dO_i, O_i>
    float *stat_mlog2;     // (H, n_q): m_i * log2(e)
    float *stat_linv;      // (H, n_q): 1 / l_i
    float *dq_part;        // (q_splits, H, n_q, D) when q_splits > 1
    float *dk_part;        // (k_splits, H, n_k, D) when k_splits > 1
    float *dv_part;
    int q_tiles, k_tiles;  // tiles per (head, sequence) for the dQ / dKdV kernels
    int q_splits;          // key-range splits of the dQ reduction
    int k_splits;          // query-range splits of the dK/dV reduction
    // fp16/bf16 varlen: the forward's sorted work list of tile pairs (same
    // layout as FwdParams::sched), written into the workspace before the
    // dK/dV and dQ launches; null for the natural grid.
    const int32_t *sched;
    int sched_max;
    int grid_k;            // fp16/bf16: blocks of the one launch that run dK/dV items
    // fp16/bf16 causal, one split: each dK/dV (dQ) item runs the tiles i and
    // T-1-i of its head, so that every item holds the same work.
    int pair_k, pair_q;
};

// CSR segment softmax over given edge scores.
struct CsrParams {
    const int32_t *row_ptr, *col_idx;  // device CSR (clamped, never trusted)
    const float *scores;               // (H, nnz) f32, head stride s_sh
    int64_t s_sh;
    const void *v;                     // (H, n_src, D) with strides v_sh, v_sn
    int64_t v_sh, v_sn;
    float *o;                          // (H, n_dst, D) f32
    int64_t o_sh, o_sn;
    float *m, *l;                      // (H, n_dst)
    int H, n_dst, n_src, nnz;
    int heads_by_xcd;  // 1: workgroup -> (head, rows) mapped per XCD (H divides 8, or 8 divides H)
    int row_blocks;    // workgroups of kCsrWaves rows per head
};

struct ReduceParams {
    const float *part;     // (splits, H, n, D) contiguous
    void *out;             // (H, n, D) with strides out_sh, out_sn
    int64_t out_sh, out_sn;
    int H, n, splits;
};

// Up to three split reductions (dK, dV, dQ) in one launch: workgroup b serves
// reduction k while b < end[k].
struct Reduce3 {
    ReduceParams r[3];
    int64_t end[3];  // cumulative workgroup counts
    int count;
    // The reduction of workgroup b; b becomes its index within that reduction.
    __device__ int which(int64_t &b) const {
        int k = 0;
        while (k + 1 < count && b >= end[k]) ++k;
        if (k > 0) b -= end[k - 1];
        return k;
    }
};

}  // namespace osattn
