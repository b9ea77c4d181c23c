/*
 * thdcp.h -- C ABI of libthdcp: one context-parallel (CP) rank's share of
 * causal self-attention over THD-packed variable-length documents, for
 * AMD Instinct MI355X (gfx950).
 *
 * Pages the operations follow (cited by title and section):
 *   [AG]  "[PyTorch] Add no-load-balance THD all-gather CP"
 *   [A2A] "[PyTorch] Extend no-load-balance CP to the a2a comm type"
 *   [PAD] "[PyTorch][Attention] THD P2P context-parallel regression when padded
 *          cu_seqlens are value-equal but not object-identical"
 *
 * Conventions for every entry point
 *   - Device buffers are owned by the caller. The library never allocates,
 *     frees or keeps device memory; the plan's device tables and the backward
 *     scratch live in caller-provided workspaces whose sizes the plan reports.
 *   - "stream" is a hipStream_t passed as void* (NULL = the default stream).
 *     Device work is only enqueued on it; no call copies device memory back
 *     to the host, and none synchronizes with the device except
 *     thdcp_plan_upload when 64 earlier uploads are still queued (see there).
 *   - Tensors are row-major THD [rows, H, D] with D contiguous (bshd with
 *     batch 1 is the same memory as THD with one document). Q/K/V/O/dO are
 *     bfloat16; LSE, the backward scratch and dQ/dK/dV are float32.
 *   - cu_seqlens / cu_seqlens_padded are int32 [B+1]: cumulative actual and
 *     cumulative physical (padded) lengths. Padding of a document sits at its
 *     end. A NULL cu_seqlens means "equal to cu_seqlens_padded".
 *   - Errors: every call returns a thdcp_status_t; on a non-OK status nothing
 *     was enqueued and thdcp_last_error() gives a message (thread-local).
 *     Invalid metadata is reported, never trapped on the device.
 */
#ifndef THDCP_H
#define THDCP_H

#include <stddef.h>
#include <stdint.h>

/* Entry points are the library's only exported symbols (it is built with
 * hidden default visibility). */
#define THDCP_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

/* Token partition strategy ([AG] "How to use", "What changed"). */
typedef enum {
  THDCP_DUAL_CHUNK_SWAP = 0, /* every padded doc cut into 2*cp_size chunks;
                                rank r holds chunks r and 2*cp_size-1-r */
  THDCP_NO_LOAD_BALANCE = 1  /* rank r holds physical rows
                                [r*s_local, (r+1)*s_local), s_local = T/cp_size */
} thdcp_strategy_t;

/* Row order of the full K/V given to the attention calls, and of the dK/dV
 * partials they return.
 *   THDCP_KV_GLOBAL: global (document) order, i.e. after the restore of
 *     [AG] sequence diagram ("restore K/V"); dK/dV come back in global order
 *     and are unrestored by the caller before the reduce-scatter.
 *   THDCP_KV_RANK_MAJOR: the order the all-gather delivers -- rank 0's local
 *     rows, then rank 1's, ... (row p is global row idx[p] of the all-ranks
 *     permutation, thd_partition_index with rank = -1). The kernels read K/V
 *     rows and write dK/dV rows through the plan's map from global row to
 *     rank-major position, so the restore before attention and the unrestore
 *     after it are fused into their loads and stores, and dK/dV come back in
 *     the order the reduce-scatter sends. Under NO_LOAD_BALANCE the two orders
 *     are the same ([A2A] body: the reorder copy disappears). */
typedef enum {
  THDCP_KV_GLOBAL = 0,
  THDCP_KV_RANK_MAJOR = 1
} thdcp_kv_layout_t;

typedef enum {
  THDCP_OK = 0,
  THDCP_ERR_ARG = 1,         /* bad pointer, size or flag combination */
  THDCP_ERR_LAYOUT = 2,      /* cu_seqlens / divisibility rules broken */
  THDCP_ERR_UNSUPPORTED = 3, /* window, head_dim or other unsupported setting */
  THDCP_ERR_HIP = 4          /* a HIP launch or copy failed */
} thdcp_status_t;

/* Message for the last non-OK status on this thread ("" if none). */
THDCP_API
const char* thdcp_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
THDCP_API
int32_t thdcp_version(void);

/*
 * Validate THD metadata and detect inter-sequence padding by value.
 * [AG] "Why" / "Scope and constraints": DUAL_CHUNK_SWAP needs every padded
 * length divisible by 2*cp_size and T == cu_seqlens_padded[B];
 * NO_LOAD_BALANCE needs only T divisible by cp_size ([A2A] body); each
 * window side is >= 0 or -1 (see thdcp_attn_desc). [PAD] "Expected
 * behavior": padding is present iff
 * some document's actual length is below its padded length or
 * T > cu_seqlens_padded[B] -- decided from the values, never from whether the
 * two arrays are the same object.
 *   pad_between_seqs: -1 = detect, 0 = caller asserts none (an error if the
 *   values show padding), 1 = caller asserts padding (accepted either way).
 *   padding_present_out (nullable): 1 if padding exists, else 0.
 * Host pointers only; no device work.
 */
THDCP_API
thdcp_status_t thdcp_validate(const int32_t* cu_seqlens_host,
                              const int32_t* cu_seqlens_padded_host, int32_t B,
                              int64_t T, int32_t cp_size, int32_t rank,
                              thdcp_strategy_t strategy, int32_t window_left,
                              int32_t window_right, int32_t pad_between_seqs,
                              int32_t* padding_present_out);

/*
 * Partition index ([AG] "What changed", "Why"; [A2A] body): for local row m of
 * `rank`, idx_out[m] is the global physical row it holds (int32 [T/cp_size]).
 * rank == -1 writes every rank's indices rank-major (int32 [T]): the
 * permutation that restores an all-gathered buffer to global order.
 * cu_seqlens_padded_host (nullable) is used only to validate; the kernel reads
 * cu_seqlens_padded_dev (int32 [B+1], device). Without the host copy the call
 * is not validated against the layout rules of thdcp_validate: it checks only
 * what needs no host data (sizes, rank, strategy, and DUAL_CHUNK_SWAP with
 * B == 0 and T > 0), and the caller guarantees the rest. A device array that
 * breaks them gives wrong indices with no error, but the kernel still stays
 * inside its buffers.
 */
THDCP_API
thdcp_status_t thd_partition_index(const int32_t* cu_seqlens_padded_host,
                                   const int32_t* cu_seqlens_padded_dev, int32_t B,
                                   int64_t T, int32_t cp_size, int32_t rank,
                                   thdcp_strategy_t strategy, int32_t* idx_out_dev,
                                   void* stream);

/*
 * Row gather: dst[m, :] = src[idx[m], :] for m in [0, n), rows of row_bytes
 * bytes (any dtype: bf16 Q/K/V rows, fp32 gradient rows, int64 token ids).
 * This is the per-rank slicing of [AG] "How to use" and the K/V restore /
 * dK-dV unrestore of the [AG] sequence diagram. idx values outside
 * [0, n_src) give an all-zero dst row. src and dst must not overlap.
 * row_bytes % 16 == 0 takes a 16-byte vector path.
 */
THDCP_API
thdcp_status_t thd_gather(const void* src_dev, int64_t n_src, const int32_t* idx_dev,
                          int64_t n, int64_t row_bytes, void* dst_dev, void* stream);

/*
 * Row scatter: dst[idx[m], :] = src[m, :] for m in [0, n). idx values outside
 * [0, n_dst) are skipped. Duplicate idx values race (last writer unspecified).
 */
THDCP_API
thdcp_status_t thd_scatter(const void* src_dev, int64_t n, const int32_t* idx_dev,
                           int64_t row_bytes, void* dst_dev, int64_t n_dst, void* stream);

/*
 * The same gather / scatter applied to 1..4 tensors that share the index, the
 * row count and the row size, in one launch (e.g. the K and V restore, the
 * local Q and dO slices, the dK and dV unrestore). src_list and dst_list are
 * host arrays of n_tensors device pointers; per tensor the behaviour is that
 * of thd_gather / thd_scatter. A move of zero rows (n == 0) succeeds without
 * looking at the pointers and enqueues nothing.
 */
THDCP_API
thdcp_status_t thd_gather_batched(int32_t n_tensors, const void* const* src_list, int64_t n_src,
                                  const int32_t* idx_dev, int64_t n, int64_t row_bytes,
                                  void* const* dst_list, void* stream);
THDCP_API
thdcp_status_t thd_scatter_batched(int32_t n_tensors, const void* const* src_list, int64_t n,
                                   const int32_t* idx_dev, int64_t row_bytes,
                                   void* const* dst_list, int64_t n_dst, void* stream);

/*
 * Local layout work around the all-to-all exchange ([A2A] body and diagram).
 * Before attention every rank sends head group c of each of its n_tokens
 * local tokens to rank c; after attention the exchange runs the other way.
 * Each token row is cp_size equal head groups of group_bytes bytes
 * (group_bytes = H / cp_size * D * sizeof(element)).
 *
 * thd_a2a_pack:   src [n_tokens, cp_size, G] -> dst [cp_size, n_tokens, G],
 *                 dst[c, m, :] = src[m, c, :]; dst block c is the contiguous
 *                 send buffer for rank c.
 * thd_a2a_unpack: src [cp_size, n_tokens, G] -> dst [n_tokens, cp_size, G],
 *                 dst[m, c, :] = src[c, m, :]; the inverse of the pack (after
 *                 the return exchange, block c holds head group c).
 *
 * Rank-major order after the forward exchange equals global order under
 * NO_LOAD_BALANCE; under DUAL_CHUNK_SWAP it is restored with
 * thd_scatter_batched by the all-ranks permutation of thd_partition_index
 * (rank = -1), and undone after attention with thd_gather_batched by the same
 * permutation. 1..4 tensors of the same shape move in one launch; src_list and
 * dst_list are host arrays of device pointers; src and dst must not overlap.
 * n_tokens * cp_size must be below 2^31; n_tokens == 0 succeeds without
 * looking at the pointers and enqueues nothing.
 */
THDCP_API
thdcp_status_t thd_a2a_pack(int32_t n_tensors, const void* const* src_list, int64_t n_tokens,
                            int32_t cp_size, int64_t group_bytes, void* const* dst_list,
                            void* stream);
THDCP_API
thdcp_status_t thd_a2a_unpack(int32_t n_tensors, const void* const* src_list, int64_t n_tokens,
                              int32_t cp_size, int64_t group_bytes, void* const* dst_list,
                              void* stream);

/* ------------------------------------------------------------------------
 * Dense layouts ([A2A] body: flat a2a is tested over bshd, sbhd and THD).
 * Attention is independent per (batch element, head), so a dense batch is
 * passed as a THD view of the same memory, with no copy:
 *   bshd [B, S, H, D]: B documents of S tokens (cu_seqlens = cu_seqlens_padded
 *                      = {0, S, 2S, ...}), H heads;
 *   sbhd [S, B, H, D]: one document of S tokens (cu_seqlens = {0, S}), B*H
 *                      heads -- the row of position s holds every batch
 *                      element's heads.
 * CP shards the sequence of every batch element. For sbhd under either
 * strategy, and for bshd under DUAL_CHUNK_SWAP (or B = 1), that is exactly
 * the THD partition of the view. bshd with B > 1 under NO_LOAD_BALANCE is
 * not (the THD partition would cut the packed B*S rows): pass it as sbhd.
 * The a2a pack/unpack around an sbhd batch takes the [S*B, H, D] row view
 * (heads split per batch element; dual chunks of that one-document view are
 * whole sequence positions).
 * ---------------------------------------------------------------------- */

/* ------------------------------------------------------------------------
 * Rank plan: the THD metadata of one rank ([AG] sequence diagram "partition
 * and build THD metadata"), built once per batch on the host and shared by
 * forward and backward so both use the same token layout ([AG] "What changed":
 * the strategy is captured for backward). It holds the per-rank valid lengths
 * ([PAD] get_cu_seqlens_on_cp_rank), the forward query-tile and backward
 * key-tile work lists (tiles wholly outside the document / causal mask are
 * never listed) and the key-row ranges that no local query attends.
 * ---------------------------------------------------------------------- */
typedef struct thdcp_plan* thdcp_plan_t;

typedef struct {
  const int32_t* cu_seqlens_host;        /* [B+1] host; NULL = cu_seqlens_padded */
  const int32_t* cu_seqlens_padded_host; /* [B+1] host */
  int32_t B;
  int64_t T;                 /* physical THD rows of the full (gathered) K/V */
  int32_t cp_size;
  int32_t rank;
  thdcp_strategy_t strategy;
  int32_t H;                 /* heads of Q, K and V (self-attention, equal) */
  int32_t D;                 /* head dim: 64 or 128 */
  float softmax_scale;       /* <= 0 selects 1/sqrt(D) */
  int32_t window_left;       /* key band of a real query at document position  */
  int32_t window_right;      /* p: real keys at [p - left, p + right]; -1 = no
                                bound. (-1, 0) causal (the default; every causal
                                mask type, queries and keys sharing one layout),
                                (-1, -1) the whole document (padding-only mask),
                                (w, 0) a causal sliding window ([A2A] body:
                                after the a2a exchange every mask type and
                                window size stays valid). P2P plans: (-1, 0). */
  int32_t pad_between_seqs;  /* -1 detect by value, 0 none, 1 present */
  int32_t kv_layout;         /* thdcp_kv_layout_t of K/V in and dK/dV out */
  int32_t p2p;               /* 1: also build the P2P ring step tables
                                (cp_attn_fwd_step / cp_attn_bwd_step) */
  int32_t max_key_splits;    /* key walks of the forward / dQ query tiles:
                                0 = the plan splits the walks longer than the
                                balanced load of a full MI355X when the
                                longest is 1.75x that load or more (few heads
                                over long causal documents), 1 = never split,
                                n >= 2 = split from the balanced load on, at
                                most n parts (capped at 8). Results are
                                deterministic either way. */
} thdcp_attn_desc;

typedef struct {
  int64_t n_local;           /* T / cp_size local rows */
  int64_t causal_pairs;      /* allowed (query,key) pairs per head */
  int64_t touched_rows;      /* key rows attended by >= 1 local query */
  int64_t untouched_rows;    /* T - touched_rows */
  int32_t padding_present;   /* by value, see thdcp_validate */
  int32_t n_fwd_tiles;       /* query tiles of the forward / dQ launches */
  int32_t n_bwd_tiles;
  int32_t n_zero_ranges;     /* untouched key-row ranges */
  size_t workspace_bytes;    /* device bytes thdcp_plan_upload needs */
  size_t bwd_scratch_bytes;  /* device bytes cp_attn_bwd needs as scratch */
  int32_t n_split_tiles;     /* query tiles whose key walk is split */
  int32_t n_fwd_parts;       /* workgroups per head of a forward / dQ launch */
  int32_t fwd_tile_rows;     /* query rows per forward / dQ tile: 256 where the
                                average local query walks >= 4096 keys (not
                                P2P plans), else 128 */
  int32_t bwd_tile_keys;     /* keys per dK/dV tile: 256 where fwd_tile_rows is
                                256, else 128 */
} thdcp_plan_info;

/* Build a plan on the host. *plan_out receives a host object the caller
 * releases with thdcp_plan_destroy. No device work. Returns
 * THDCP_ERR_UNSUPPORTED when one document's rows, or the local share's rows,
 * of bf16 [H, D] reach 2 GiB (the kernels address them with 32-bit buffer
 * offsets), or, for THDCP_KV_RANK_MAJOR, when all T rows do. */
THDCP_API
thdcp_status_t thdcp_plan_create(const thdcp_attn_desc* desc, thdcp_plan_t* plan_out);
THDCP_API
thdcp_status_t thdcp_plan_get_info(thdcp_plan_t plan, thdcp_plan_info* info_out);
/* Per-document count of real tokens this rank holds (int32 [B], host). */
THDCP_API
thdcp_status_t thdcp_plan_local_seqlens(thdcp_plan_t plan, int32_t* out_host);
/* Copy the plan's device tables into the caller's workspace (device,
 * >= workspace_bytes, 256-byte aligned) with one async host-to-device copy on
 * `stream`. The plan keeps the pointer; the workspace must stay alive and
 * unmodified while forward/backward calls using the plan are in flight.
 * Past the tables it holds the split key walks' counters (uploaded as zero,
 * left at zero by every launch) and their partial results, and, for plans
 * with fwd_tile_rows 256 and head dim 128, V transposed (H * 128 * pitch
 * bf16, pitch = T rounded up to 64, plus 128), which cp_attn_fwd writes from
 * v before its attention launch. So the plan's forward and dQ launches must
 * not overlap: enqueue calls that use one workspace on one stream (or order
 * them). The copy covers the tables and counters only.
 * Tables up to 1 MiB are first copied into a page-locked staging slot the
 * library keeps for the life of the process (1 MiB each, allocated 16 at a
 * time: 16 on the first upload, 16 more whenever every slot still feeds a
 * copy the GPU has not run, up to 64 slots), so the plan may be destroyed
 * right after this call. Like every other call it does not wait for the
 * device, with one exception: when 64 uploads are still queued on the GPU,
 * the next one waits until the oldest of them has run. Larger tables are
 * copied from the plan itself, which must then outlive the copy. */
THDCP_API
thdcp_status_t thdcp_plan_upload(thdcp_plan_t plan, void* workspace_dev, size_t bytes,
                                 void* stream);
THDCP_API
void thdcp_plan_destroy(thdcp_plan_t plan);

/*
 * Forward ([AG] "Why": DUAL_CHUNK_SWAP's two attention steps and
 * NO_LOAD_BALANCE's one are all query tiles of this single launch; the mask is
 * the cp_size = 1 mask, [A2A] body). Each real local query g attends the keys
 * j of its own document with j <= g (in general: the real keys of its
 * document inside the plan's window):
 *   O = softmax(scale * q K^T) V,   LSE = log sum exp(scale * q K^T).
 *   q_local  bf16 [n_local, H, D]   local queries in local row order
 *   k, v     bf16 [T, H, D]         full K/V in the plan's kv_layout
 *   o_local  bf16 [n_local, H, D]   written for every local row
 *   lse      fp32 [H, n_local]      natural log; -inf on padding rows
 * Padding rows get O = 0. Padding key rows are never read into a product.
 * The probabilities enter P V as bf16; at head dim 128 the sum that normalises
 * O and enters LSE is taken over those same bf16 values (on the matrix cores),
 * so LSE carries their rounding: within log(1 + 2^-8) of the exact value,
 * measured up to 2.3e-3. At head dim 64 the sum is taken in fp32.
 * Plans with fwd_tile_rows 256 and head dim 128 first write V^T into the
 * workspace (one pass over v; keys no local query attends, padding included,
 * as 0) and stage V^T tiles instead of V rows.
 * A query tile whose key walk the plan split (max_key_splits) is computed by
 * several workgroups of the same launch; the last to finish merges their
 * (max, sum, accumulator) states in key order, so the output is
 * bit-identical from run to run.
 */
THDCP_API
thdcp_status_t cp_attn_fwd(thdcp_plan_t plan, const void* q_local, const void* k,
                           const void* v, void* o_local, float* lse, void* stream);

/*
 * Backward of cp_attn_fwd for loss gradient dO ([AG] sequence diagram: the
 * dK/dV produced here are the partials that are unrestored for the
 * reduce-scatter).
 *   o_local, lse  outputs of cp_attn_fwd;  d_o bf16 [n_local, H, D]
 *   dq      fp32 [n_local, H, D]   fully written (padding rows 0)
 *   k, v    bf16 [T, H, D] in the plan's kv_layout
 *   dk, dv  fp32 [T, H, D]         this rank's partial, in the plan's
 *                                  kv_layout: rows attended by at least one
 *                                  local query are written
 *                                  (accumulate_dkv = 1: added to dk/dv)
 *   zero_untouched = 1: also write 0 to every other row of dk/dv -- padding
 *   rows, the buffer tail and keys no local query attends. The zeroing runs
 *   only when the plan has such rows, so a layout with no tail costs nothing
 *   ([PAD] "Expected behavior": gate tail zeroing on the metadata).
 *   zero_untouched and accumulate_dkv are mutually exclusive.
 *   scratch  device, >= bwd_scratch_bytes, 256-byte aligned.
 * Two launches: the dQ kernel, which also computes delta = rowsum(dO * O)
 * into scratch and whose grid ends with the zeroing workgroups when
 * zero_untouched = 1 and the plan has such rows, then the dK/dV kernel.
 * Every output row is written by exactly one workgroup (a split dQ walk's
 * parts are summed in key order by the last part to finish; a counter
 * atomic only decides which part that is), so dQ, dK and dV are
 * bit-identical from run to run.
 */
THDCP_API
thdcp_status_t cp_attn_bwd(thdcp_plan_t plan, const void* q_local, const void* k,
                           const void* v, const void* o_local, const float* lse,
                           const void* d_o, float* dq, float* dk, float* dv,
                           int32_t zero_untouched, int32_t accumulate_dkv, void* scratch,
                           size_t scratch_bytes, void* stream);

/*
 * cp_attn_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same launches and results as cp_attn_bwd, with its scratch (delta, fp32
 * [H, n_local]) in a fixed 8 MiB device array of the library instead of a
 * caller buffer. The call allocates nothing and takes no workspace argument;
 * the plan's own workspace (thdcp_plan_upload) is still used as by
 * cp_attn_bwd.
 *   Limit: n_local * H <= 2,097,152 (2^21 floats); a larger plan gets
 *   THDCP_ERR_UNSUPPORTED before anything is enqueued.
 *   Each GPU holds its own copy of the array until the process ends, and
 *   every call on that GPU shares it: calls that overlap on one GPU (on two
 *   streams, or from two threads) race. Calls enqueued on one stream are
 *   ordered and safe. The first call on a device looks up the array's device
 *   address (no allocation).
 */
THDCP_API
thdcp_status_t cp_attn_bwd_noalloc(thdcp_plan_t plan, const void* q_local, const void* k,
                                   const void* v, const void* o_local, const float* lse,
                                   const void* d_o, float* dq, float* dk, float* dv,
                                   int32_t zero_untouched, int32_t accumulate_dkv,
                                   void* stream);

/*
 * The backward as separate launches, for callers that schedule or time them
 * one by one. Calling preprocess, dkdv, dq and thdcp_zero_untouched in this
 * order on one stream computes the gradients cp_attn_bwd computes (which
 * folds the preprocess and the zeroing into its dQ launch); delta is summed
 * in a different order there, so the two agree to rounding, not bit for bit.
 *   cp_attn_bwd_preprocess: delta[h, m] = sum_d dO[m,h,d] * O[m,h,d] (fp32,
 *     [H, n_local], into scratch).
 *   cp_attn_bwd_dkdv: the dK/dV partials (key-tile-major; written, or added
 *     when accumulate_dkv = 1, for every attended key row).
 *   cp_attn_bwd_dq: dQ for every local row (query-tile-major; padding rows 0).
 *     dkdv and dq only read delta, so they may run in either order.
 *   thdcp_zero_untouched: writes 0 to every dk/dv row no local query attends;
 *     enqueues nothing when the plan has no such row.
 */
THDCP_API
thdcp_status_t cp_attn_bwd_preprocess(thdcp_plan_t plan, const void* o_local, const float* lse,
                                      const void* d_o, void* scratch, size_t scratch_bytes,
                                      void* stream);
THDCP_API
thdcp_status_t cp_attn_bwd_dkdv(thdcp_plan_t plan, const void* q_local, const void* k,
                                const void* v, const float* lse, const void* d_o, float* dk,
                                float* dv, int32_t accumulate_dkv, const void* scratch,
                                size_t scratch_bytes, void* stream);
THDCP_API
thdcp_status_t cp_attn_bwd_dq(thdcp_plan_t plan, const void* q_local, const void* k,
                              const void* v, const float* lse, const void* d_o, float* dq,
                              const void* scratch, size_t scratch_bytes, void* stream);
THDCP_API
thdcp_status_t thdcp_zero_untouched(thdcp_plan_t plan, float* dk, float* dv, void* stream);

/* ------------------------------------------------------------------------
 * P2P (ring) context parallelism ([PAD] "Describe the bug": the P2P path runs
 * a rank's attention in steps over its peers' K/V, with per-step sequence
 * metadata and gradient tails to clear). At ring step i, rank `rank` works on
 * the K/V that rank src = (rank - i) mod cp_size holds; the step results are
 * merged through their log-sum-exp, all at once with thdcp_lse_merge_parts
 * once every step has run, or step by step with thdcp_lse_merge. These calls need a
 * plan made with p2p = 1: every step's tiles come from that one plan, built
 * once per batch, so no step launches metadata work, and a step's gradient
 * tail is zeroed only when the plan shows one.
 * ---------------------------------------------------------------------- */

/*
 * Attention of the local queries against the keys rank src_rank holds (same
 * document, key <= query):
 *   k_src, v_src  bf16 [n_local, H, D]  rank src's local K/V, in its local
 *                                       row order (thd_partition_index order)
 *   o_part        bf16 [n_local, H, D]  softmax over this step's keys times V;
 *                                       0 on rows with no key in the step
 *   lse_part      fp32 [H, n_local]     this step's LSE; -inf on such rows
 */
THDCP_API
thdcp_status_t cp_attn_fwd_step(thdcp_plan_t plan, int32_t src_rank, const void* q_local,
                                const void* k_src, const void* v_src, void* o_part,
                                float* lse_part, void* stream);

/*
 * Fold one step's (o_part bf16 [n, H, D], lse_part fp32 [H, n]) into the
 * running result (o_acc fp32 [n, H, D], lse_acc fp32 [H, n]):
 *   lse = log(exp(lse_acc) + exp(lse_part)),
 *   o_acc = (exp(lse_acc) o_acc + exp(lse_part) o_part) / exp(lse).
 * first = 1 starts the accumulation (o_acc, lse_acc are only written). o_out
 * (bf16 [n, H, D], nullable) also receives the merged output rounded to bf16,
 * for the last step. Rows that are -inf in both stay O = 0, LSE = -inf. One
 * elementwise launch; n == 0 enqueues nothing.
 */
THDCP_API
thdcp_status_t thdcp_lse_merge(int64_t n, int32_t H, int32_t D, const void* o_part,
                               const float* lse_part, float* o_acc, float* lse_acc,
                               int32_t first, void* o_out, void* stream);

/*
 * Merge every step's result at once: with the parts' LSEs l_p and
 * M = max_p l_p,
 *   lse = M + log sum_p exp(l_p - M),
 *   o   = sum_p exp(l_p - M) o_p / sum_p exp(l_p - M),
 * summed in part order (bit-identical from run to run).
 *   o_parts    bf16 [parts, n, H, D]  step p's o_part at o_parts + p*n*H*D
 *   lse_parts  fp32 [parts, H, n]     step p's lse_part
 *   o_out      bf16 [n, H, D]         the merged output
 *   lse_out    fp32 [H, n]            the merged LSE (nullable)
 * Rows that are -inf in every part get O = 0, LSE = -inf. One elementwise
 * launch that reads each part once, in place of parts merges into an fp32
 * accumulator that is read and written at every step. n == 0 enqueues
 * nothing.
 */
THDCP_API
thdcp_status_t thdcp_lse_merge_parts(int64_t n, int32_t H, int32_t D, int32_t parts,
                                     const void* o_parts, const float* lse_parts, void* o_out,
                                     float* lse_out, void* stream);

/*
 * Backward of one step with the softmax of the whole key set: lse is the
 * merged LSE, scratch holds delta of the merged output (cp_attn_bwd_preprocess
 * on the merged O and dO).
 *   dq      fp32 [n_local, H, D]  written (accumulate_dq = 0, the first step)
 *                                 or added to
 *   dk_src, dv_src  fp32 [n_local, H, D], rank src's local row order: this
 *           rank's partial for rank src's keys (what the ring sends back);
 *           rows attended by a local query are written. zero_untouched = 1
 *           also writes 0 to the other rows, only when the plan has such rows.
 * Two launches (dQ with the zeroing workgroups, then dK/dV); no atomics.
 */
THDCP_API
thdcp_status_t cp_attn_bwd_step(thdcp_plan_t plan, int32_t src_rank, const void* q_local,
                                const void* k_src, const void* v_src, const float* lse,
                                const void* d_o, const void* scratch, size_t scratch_bytes,
                                float* dq, int32_t accumulate_dq, float* dk_src, float* dv_src,
                                int32_t zero_untouched, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* THDCP_H */
