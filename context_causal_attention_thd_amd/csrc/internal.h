// Internal definitions shared by the host planner and the gfx950 kernels.
// Not part of the public ABI (include/thdcp.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "thdcp.h"

namespace thdcp {

// Sets the thread's thdcp_last_error() text and returns st (capi.cpp).
thdcp_status_t report_error(thdcp_status_t st, const char* msg);

// Forward work item: up to kFwdBM (or kFwdBMLong) consecutive local rows that
// lie in one contiguous run of global rows of one document (a DUAL_CHUNK_SWAP chunk or a
// NO_LOAD_BALANCE document piece), so row r of the tile is global row g0 + r.
// The keys it attends are walked in doc-aligned blocks over [ks0, ke0), then
// over [ks1, ke1) (either range may be empty): the whole causal range
// [doc start, last real row + 1) for the all-gather pass; for one P2P step,
// the parts of it that the step's source rank holds (at most two
// DUAL_CHUNK_SWAP chunks of the document).
//
// Split key walk: when nparts > 1 the tile's key tiles are walked by nparts
// workgroups, part p taking the p-th of nparts equal runs of them in walk
// order (so only the last part reaches the diagonal). Each part writes its
// partial result to scratch slot `slot + part`; the one that finishes last
// (counted on counter `group`) combines all of them in part order, so the
// result does not depend on which part finished last.
struct FwdTile {
  int32_t m0;        // first local row
  int32_t n;         // rows in the tile (<= the plan's tile rows)
  int32_t g0;        // global row of m0
  int32_t e;         // end of the document's real tokens (a + actual length)
  int32_t ks0, ke0;  // first key range
  int32_t ks1, ke1;  // second key range
  int32_t part, nparts;
  int32_t slot, group;
};

// Backward work item: key rows [k0, k1) of one document (all attended by at
// least one local query) and the local query rows [m_lo, m_hi) that attend
// them. Those rows are real tokens of the same document in ascending global
// order; the global row of local row m is m + dg_a below m_split, m + dg_b
// from m_split on (the two DUAL_CHUNK_SWAP chunks of the document).
struct BwdTile {
  int32_t k0, k1;
  int32_t m_lo, m_hi;
  int32_t m_split;
  int32_t dg_a, dg_b;
  int32_t pad0;
};

// Rows [r0, r1) of dK/dV that no local query attends; `before` is the number
// of such rows in all earlier ranges (prefix sum for the zeroing kernel).
struct ZeroRange {
  int32_t r0, r1;
  int32_t before;
  int32_t pad0;
};

constexpr int kFwdBM = 128;      // query rows per forward / dQ workgroup
constexpr int kFwdBMLong = 256;  // the same for plans whose walks are long
constexpr int kFwdBN = 64;       // keys per forward K/V tile
constexpr int kBwdBN = 128;      // keys per backward workgroup (4 waves x 32)
constexpr int kBwdBNLong = 256;  // the same for plans whose walks are long (8 x 32)

// Scratch of split key walks: per (slot, head) kSplitFloats(D, rows) floats
// hold one part's partial result for a tile of `rows` query rows (forward:
// rows x D accumulators, then a running max and row-sum share per 16-row block
// and lane; dQ: rows x D accumulators), in the owning kernel's lane order;
// cnt[group * H + head] counts the parts that have finished (0 between
// launches).
constexpr int64_t kSplitFloats(int D, int rows) { return (int64_t)rows * (D + 8); }
struct SplitWs {
  int32_t* cnt;
  float* part;
};

// Kernel launchers (defined in the .hip files). All enqueue on `stream`.
hipError_t launch_partition(const int32_t* cup, int32_t B, int64_t T, int32_t cp,
                            int32_t rank, int32_t strategy, int32_t* out, int64_t n_out,
                            hipStream_t stream);
constexpr int kMaxMoveTensors = 4;  // tensors one gather/scatter launch can move
hipError_t launch_gather(int32_t n_tensors, const void* const* srcs, int64_t n_src,
                         const int32_t* idx, int64_t n, int64_t row_bytes, void* const* dsts,
                         hipStream_t stream);
hipError_t launch_scatter(int32_t n_tensors, const void* const* srcs, int64_t n,
                          const int32_t* idx, int64_t row_bytes, void* const* dsts,
                          int64_t n_dst, hipStream_t stream);
// Head-group pack ([n, cp, G] -> [cp, n, G]) or its inverse, G = group_bytes.
hipError_t launch_a2a(int32_t n_tensors, const void* const* srcs, int64_t n_tokens, int32_t cp,
                      int64_t group_bytes, void* const* dsts, bool unpack, hipStream_t stream);
// bytes (a multiple of 16) from src (device-readable, e.g. page-locked host
// memory) to dst, by a kernel on `stream`.
hipError_t launch_copy16(const void* src, void* dst, int64_t bytes, hipStream_t stream);
// K/V row addressing shared by the attention and zeroing launches: global key
// g sits at row (map ? map[g] : g) - sub of k, v (and dk, dv), which hold
// `rows` rows. map is the rank-major map (null: identity); sub != 0 addresses
// one rank's local block (a P2P step's source rank).
// Key band of the attention mask: a real query at global row g attends keys
// [g - wl, g + wr] of its document's real rows (the plan's tile ranges keep
// the keys inside the document). kUnbounded stands for "no bound" on a side:
// with T below 2^30 every g +- kUnbounded stays inside int32. The causal
// mask is {kUnbounded, 0}; `causal` says so, which lets the dK/dV kernel skip
// the lower-bound test.
constexpr int32_t kUnbounded = 1 << 30;
struct Band {
  int32_t wl, wr;
  bool causal;
};
struct KvRows {
  const int32_t* map;
  int64_t sub;
  int64_t rows;
};

hipError_t launch_zero_rows(const ZeroRange* ranges, int32_t n_ranges, int64_t total_rows,
                            KvRows kv, int64_t row_floats, float* a, float* b,
                            hipStream_t stream);
// Fold (o_part bf16, lse_part) into (o_acc fp32, lse_acc); see thdcp_lse_merge.
hipError_t launch_lse_merge(int64_t n, int32_t H, int32_t D, const void* o_part,
                            const float* lse_part, float* o_acc, float* lse_acc, int32_t first,
                            void* o_out, hipStream_t stream);
// Merge `parts` step results (o_parts bf16 [parts, n, H, D], lse_parts fp32
// [parts, H, n]) into o_out bf16 [n, H, D] and lse_out fp32 [H, n] (nullable).
hipError_t launch_lse_merge_parts(int64_t n, int32_t H, int32_t D, int32_t parts,
                                  const void* o_parts, const float* lse_parts, void* o_out,
                                  float* lse_out, hipStream_t stream);
hipError_t launch_bwd_prep(const void* o, const void* d_o, const float* lse, float* delta,
                           int64_t n_local, int32_t H, int32_t D, hipStream_t stream);
// rows: query rows per tile of the plan (kFwdBM or kFwdBMLong); the forward
// and dQ launches pick their wave shape from it. vt (optional, rows ==
// kFwdBMLong and D == 128 only): V^T written by launch_v_transpose for the
// same K/V, pitch vt_pitch; the forward then stages V^T tiles instead of V.
hipError_t launch_attn_fwd(const FwdTile* tiles, int32_t n_tiles, int32_t H, int32_t D,
                           int32_t rows, const void* q, const void* k, const void* v, KvRows kv,
                           Band band, void* o, float* lse, int64_t n_local, float scale,
                           SplitWs split, const void* vt, int32_t vt_pitch, hipStream_t stream);
// Key pitch of V^T for T keys: a multiple of 64 with 64 keys to spare past
// the last tile start.
int32_t vt_pitch_for(int64_t T);
// V^T [H][128][pitch] (bf16) of the kv.rows keys of V (row addressing as in
// KvRows), 0 for keys >= kv.rows and keys inside the zero ranges zr.
hipError_t launch_v_transpose(const void* v, KvRows kv, int32_t H, int32_t D,
                              const ZeroRange* zr, int32_t n_zr, void* vt, int32_t pitch,
                              hipStream_t stream);
// keys: keys per tile of the plan (kBwdBN or kBwdBNLong).
hipError_t launch_attn_bwd_dkdv(const BwdTile* tiles, int32_t n_tiles, int32_t H, int32_t D,
                                int32_t keys, const void* q, const void* k, const void* v, KvRows kv,
                                Band band, const void* d_o, const float* lse,
                                const float* delta, float* dk, float* dv, int64_t n_local,
                                float scale, int32_t accumulate, hipStream_t stream);
// Work a dQ launch carries besides dQ: workgroups at the end of its grid that
// zero the dK/dV rows no local query attends (zr/n_zr/zero_rows, rows found
// through the launch's KvRows). It is independent of dQ and fills the
// launch's tail.
struct DqExtras {
  const ZeroRange* zr = nullptr;
  int32_t n_zr = 0;
  int64_t zero_rows = 0;
  float* dk = nullptr;
  float* dv = nullptr;
};
// o (nullable): when given, delta = rowsum(dO * O) is computed by this launch
// and written to `delta` for the dK/dV kernel; otherwise `delta` is read.
// accumulate: add to dq (P2P steps after the first) instead of writing it.
hipError_t launch_attn_bwd_dq(const FwdTile* tiles, int32_t n_tiles, int32_t H, int32_t D,
                              int32_t rows, const void* q, const void* k, const void* v, KvRows kv,
                              Band band, const void* d_o, const void* o, const float* lse,
                              float* delta,
                              float* dq, int64_t n_local, float scale, int32_t accumulate,
                              SplitWs split, const DqExtras& extras, hipStream_t stream);

}  // namespace thdcp
