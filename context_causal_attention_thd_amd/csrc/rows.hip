// Row-movement and small bandwidth-bound kernels for gfx950:
//   partition index ("[PyTorch] Add no-load-balance THD all-gather CP",
//   "What changed" and "Why"), row gather / scatter (the rank slicing of its
//   "How to use" and the K/V restore / dK-dV unrestore of its sequence
//   diagram), the head-group pack / unpack around the all-to-all exchange
//   ("[PyTorch] Extend no-load-balance CP to the a2a comm type", body and
//   diagram), the gated zeroing of untouched gradient rows ("THD P2P
//   context-parallel regression ...", "Expected behavior") and the backward
//   preprocess delta = rowsum(dO * O).
//
// All of these are HBM-bound: each maps (row, 16-byte chunk) pairs onto
// consecutive lanes so that every wave issues contiguous 16-byte accesses.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace thdcp {

// ---------------------------------------------------------------------------
// Partition index
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) partition_kernel(const int32_t* __restrict__ cup,
                                                        int32_t B, int64_t T, int32_t cp,
                                                        int32_t rank, int32_t strategy,
                                                        int32_t* __restrict__ out,
                                                        int64_t n_out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_out) return;
  const int64_t s_local = T / cp;
  const int64_t r = rank >= 0 ? rank : i / s_local;
  const int64_t m = rank >= 0 ? i : i - r * s_local;
  if (strategy == 1) {  // NO_LOAD_BALANCE: contiguous physical range
    out[i] = (int32_t)(r * s_local + m);
    return;
  }
  // DUAL_CHUNK_SWAP: document j occupies local rows [cup[j]/cp, cup[j+1]/cp);
  // find the last j in [0, B) with cup[j] <= m*cp (cup[j] is a multiple of cp).
  int32_t lo = 0, hi = B - 1;
  const int64_t key = m * cp;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if ((int64_t)cup[mid] <= key) lo = mid; else hi = mid - 1;
  }
  const int64_t a = cup[lo];
  const int64_t c = ((int64_t)cup[lo + 1] - a) / (2 * cp);
  const int64_t j = m - a / cp;
  const int64_t g = j < c ? a + r * c + j : a + (2 * cp - 1 - r) * c + (j - c);
  out[i] = (int32_t)g;
}

hipError_t launch_partition(const int32_t* cup, int32_t B, int64_t T, int32_t cp, int32_t rank,
                            int32_t strategy, int32_t* out, int64_t n_out, hipStream_t stream) {
  if (B == 0 && strategy == 0) {
    // no documents: nothing to index (T must then be 0 under DUAL_CHUNK_SWAP)
    return hipSuccess;
  }
  const int threads = 256;
  const int64_t blocks = (n_out + threads - 1) / threads;
  hipLaunchKernelGGL(partition_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, cup, B, T,
                     cp, rank, strategy, out, n_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Gather / scatter of rows of arbitrary byte size
// ---------------------------------------------------------------------------
template <int VB>
struct Vec;
template <> struct Vec<16> { typedef u32x4 T; };
template <> struct Vec<8> { typedef u32x2 T; };
template <> struct Vec<4> { typedef uint32_t T; };
template <> struct Vec<2> { typedef uint16_t T; };
template <> struct Vec<1> { typedef uint8_t T; };

// One 16-byte (or narrower) chunk per thread per grid-stride step, plain
// loads and nontemporal stores, index arithmetic in 32 bits unless the launch
// has 2^32 chunks or more (WIDE). Measured on MI355X for the K+V restore of
// one 8192-row, 4 KiB-row share (134 MB moved): 5.59 TB/s with the source
// and destination rotated through more than the 256 MB last-level cache,
// 6.41 TB/s when they stay in it; four chunks per thread with nontemporal
// loads and a 64-bit division per chunk gave 5.22 / 5.65, and a plain
// device-to-device copy of the same bytes 4.74 / 6.46.
constexpr int kRowThreads = 256;

// Up to kMaxTensors tensors moved by one launch (blockIdx.y picks the tensor).
struct RowPtrs {
  const char* src[kMaxMoveTensors];
  char* dst[kMaxMoveTensors];
};

// Which row of src feeds which row of dst. The index modes read an int32
// table; the a2a modes compute the row from (n, cp) and read no table.
enum MoveMode : int {
  kGather = 0,   // dst[m] = src[idx[m]]; idx outside [0, n_other) gives a zero row
  kScatter = 1,  // dst[idx[m]] = src[m]; idx outside [0, n_other) is skipped
  kPack = 2,     // dst[c*n + m] = src[m*cp + c]  ([n, cp, G] -> [cp, n, G])
  kUnpack = 3,   // dst[m*cp + c] = src[c*n + m]  ([cp, n, G] -> [n, cp, G])
};

struct RowMap {
  const int32_t* idx;
  int64_t n_other;  // index modes: rows of the indexed tensor
  int64_t n;        // a2a modes: tokens per group
  int64_t cp;       // a2a modes: groups
};

template <int VB, int MODE, bool WIDE>
__global__ void __launch_bounds__(kRowThreads) move_rows_kernel(
    const RowPtrs ptrs, const RowMap map, uint32_t chunks_per_row, uint64_t total_chunks,
    int64_t row_bytes) {
  typedef typename Vec<VB>::T V;
  typedef typename std::conditional<WIDE, uint64_t, uint32_t>::type I;
  const char* __restrict__ src = ptrs.src[blockIdx.y];
  char* __restrict__ dst = ptrs.dst[blockIdx.y];
  const uint64_t stride = (uint64_t)gridDim.x * kRowThreads;
  for (uint64_t t = (uint64_t)blockIdx.x * kRowThreads + threadIdx.x; t < total_chunks;
       t += stride) {
    const I row = (I)t / (I)chunks_per_row;
    const uint32_t c = (uint32_t)((I)t - row * (I)chunks_per_row);
    int64_t srow, drow;
    bool load = true;
    if (MODE == kGather || MODE == kScatter) {
      const int64_t other = map.idx[row];
      const bool in = other >= 0 && other < map.n_other;
      srow = MODE == kScatter ? (int64_t)row : other;
      drow = MODE == kScatter ? (in ? other : -1) : (int64_t)row;
      load = MODE == kScatter || in;
    } else if (MODE == kPack) {
      const int64_t grp = (int64_t)row / map.n;
      srow = ((int64_t)row - grp * map.n) * map.cp + grp;
      drow = (int64_t)row;
    } else {
      const int64_t tok = (int64_t)row / map.cp;
      srow = ((int64_t)row - tok * map.cp) * map.n + tok;
      drow = (int64_t)row;
    }
    if (drow < 0) continue;
    const V val =
        load ? *reinterpret_cast<const V*>(src + srow * row_bytes + (int64_t)c * VB) : V{};
    __builtin_nontemporal_store(val,
                                reinterpret_cast<V*>(dst + drow * row_bytes + (int64_t)c * VB));
  }
}

template <int MODE, bool WIDE>
hipError_t launch_move_vb(int vb, dim3 grid, dim3 block, const RowPtrs& ptrs, const RowMap& map,
                          uint64_t cpr, uint64_t total, int64_t row_bytes, hipStream_t stream) {
#define THDCP_MOVE(VB)                                                                        \
  hipLaunchKernelGGL((move_rows_kernel<VB, MODE, WIDE>), grid, block, 0, stream, ptrs, map, \
                     (uint32_t)cpr, total, row_bytes)
  switch (vb) {
    case 16: THDCP_MOVE(16); break;
    case 8: THDCP_MOVE(8); break;
    case 4: THDCP_MOVE(4); break;
    case 2: THDCP_MOVE(2); break;
    default: THDCP_MOVE(1); break;
  }
#undef THDCP_MOVE
  return hipGetLastError();
}

// n: rows the launch walks (dst rows for gather / pack / unpack, src rows for
// scatter).
template <int MODE>
hipError_t launch_move(int32_t n_tensors, const void* const* srcs, void* const* dsts,
                       const RowMap& map, int64_t n, int64_t row_bytes, hipStream_t stream) {
  if (n_tensors < 1 || n_tensors > kMaxMoveTensors) return hipErrorInvalidValue;
  RowPtrs ptrs{};
  uintptr_t addr_bits = 0;
  for (int i = 0; i < n_tensors; ++i) {
    ptrs.src[i] = static_cast<const char*>(srcs[i]);
    ptrs.dst[i] = static_cast<char*>(dsts[i]);
    addr_bits |= reinterpret_cast<uintptr_t>(srcs[i]) | reinterpret_cast<uintptr_t>(dsts[i]);
  }
  int vb = 1;
  for (int cand : {16, 8, 4, 2}) {
    if (row_bytes % cand == 0 && (addr_bits % cand) == 0) { vb = cand; break; }
  }
  const uint64_t cpr = (uint64_t)(row_bytes / vb);
  const uint64_t total = cpr * (uint64_t)n;
  if (cpr > 0xffffffffull) return hipErrorInvalidValue;
  if (total == 0) return hipSuccess;
  uint64_t blocks = (total + kRowThreads - 1) / kRowThreads;
  if (blocks > 65536) blocks = 65536;
  const dim3 grid((unsigned)blocks, (unsigned)n_tensors), block(kRowThreads);
  if (total >= (1ull << 32)) return launch_move_vb<MODE, true>(vb, grid, block, ptrs, map, cpr, total, row_bytes, stream);
  return launch_move_vb<MODE, false>(vb, grid, block, ptrs, map, cpr, total, row_bytes, stream);
}

hipError_t launch_gather(int32_t n_tensors, const void* const* srcs, int64_t n_src,
                         const int32_t* idx, int64_t n, int64_t row_bytes, void* const* dsts,
                         hipStream_t stream) {
  const RowMap map{idx, n_src, 0, 1};
  return launch_move<kGather>(n_tensors, srcs, dsts, map, n, row_bytes, stream);
}

hipError_t launch_scatter(int32_t n_tensors, const void* const* srcs, int64_t n,
                          const int32_t* idx, int64_t row_bytes, void* const* dsts,
                          int64_t n_dst, hipStream_t stream) {
  const RowMap map{idx, n_dst, 0, 1};
  return launch_move<kScatter>(n_tensors, srcs, dsts, map, n, row_bytes, stream);
}

hipError_t launch_a2a(int32_t n_tensors, const void* const* srcs, int64_t n_tokens, int32_t cp,
                      int64_t group_bytes, void* const* dsts, bool unpack, hipStream_t stream) {
  const RowMap map{nullptr, 0, n_tokens, cp};
  const int64_t rows = n_tokens * cp;
  return unpack ? launch_move<kUnpack>(n_tensors, srcs, dsts, map, rows, group_bytes, stream)
                : launch_move<kPack>(n_tensors, srcs, dsts, map, rows, group_bytes, stream);
}

// ---------------------------------------------------------------------------
// Zero the dK/dV rows no local query attends (only launched when some exist)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) zero_rows_kernel(const ZeroRange* __restrict__ ranges,
                                                        int32_t n_ranges, uint64_t total_vec,
                                                        uint32_t vec_per_row,
                                                        const int32_t* __restrict__ kv_row,
                                                        int32_t kv_sub, float* __restrict__ a,
                                                        float* __restrict__ b) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  for (uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total_vec;
       t += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t lin = t / vec_per_row;  // index among all untouched rows
    const uint32_t c = (uint32_t)(t - lin * vec_per_row);
    int32_t lo = 0, hi = n_ranges - 1;     // last range with before <= lin
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if ((uint64_t)ranges[mid].before <= lin) lo = mid; else hi = mid - 1;
    }
    const int64_t g = ranges[lo].r0 + (int64_t)(lin - ranges[lo].before);
    const int64_t row = (kv_row ? kv_row[g] : g) - kv_sub;  // global row -> row of a and b
    const int64_t off = row * vec_per_row + c;
    reinterpret_cast<f32x4*>(a)[off] = z;
    reinterpret_cast<f32x4*>(b)[off] = z;
  }
}

hipError_t launch_zero_rows(const ZeroRange* ranges, int32_t n_ranges, int64_t total_rows,
                            KvRows kv, int64_t row_floats, float* a, float* b,
                            hipStream_t stream) {
  if (row_floats % 4 != 0) return hipErrorInvalidValue;
  const uint64_t vpr = (uint64_t)row_floats / 4;
  const uint64_t total = vpr * (uint64_t)total_rows;
  if (total == 0) return hipSuccess;
  uint64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ranges,
                     n_ranges, total, (uint32_t)vpr, kv.map, (int32_t)kv.sub, a, b);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Plan upload: a plain 16-byte copy from page-locked host memory (read by the
// GPU over the host link) into the caller's workspace. A kernel keeps the
// upload on the compute queue; a copy-engine transfer inside the stream costs
// ~15 us of idle GPU time for the queue hand-off (measured on MI355X).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) copy16_kernel(const u32x4* __restrict__ src,
                                                     u32x4* __restrict__ dst, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

hipError_t launch_copy16(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  if (bytes % 16 != 0) return hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(copy16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// P2P step merge through the log-sum-exp. D/8 lanes per (row, head), each
// taking 8 head dims (16 bytes of the bf16 step output, 32 of the fp32
// accumulator). The lanes of one (row, head) are consecutive lanes of one
// wave, so they all read lse_acc before lane 0 of the group writes it.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) lse_merge_kernel(int64_t n, int32_t H,
                                                        const bf16* __restrict__ o_part,
                                                        const float* __restrict__ lse_part,
                                                        float* __restrict__ o_acc,
                                                        float* __restrict__ lse_acc,
                                                        int32_t first, bf16* __restrict__ o_out) {
  constexpr int G = D / 8;
  const int64_t pairs = n * H;
  const int64_t pr = (int64_t)blockIdx.x * (blockDim.x / G) + threadIdx.x / G;
  if (pr >= pairs) return;
  const int sub = threadIdx.x % G;
  const int64_t m = pr / H;
  const int32_t h = (int32_t)(pr - m * H);
  const int64_t li = (int64_t)h * n + m;
  const int64_t off = pr * D + sub * 8;
  const float lp = lse_part[li];
  const bf16x8 op = load_bf16x8(o_part + off);
  f32x4* acc = reinterpret_cast<f32x4*>(o_acc + off);
  f32x4 r0, r1;
  float lnew;
  if (first) {
    for (int j = 0; j < 4; ++j) {
      r0[j] = (float)op[j];
      r1[j] = (float)op[4 + j];
    }
    lnew = lp;
  } else {
    const float la = lse_acc[li];
    const float mx = fmaxf(la, lp);
    const f32x4 a0 = acc[0], a1 = acc[1];
    if (mx == -INFINITY) {  // neither part has a key for this row
      r0 = a0;
      r1 = a1;
      lnew = -INFINITY;
    } else {
      const float wa = __expf(la - mx), wp = __expf(lp - mx);
      const float inv = 1.f / (wa + wp);
      for (int j = 0; j < 4; ++j) {
        r0[j] = (a0[j] * wa + (float)op[j] * wp) * inv;
        r1[j] = (a1[j] * wa + (float)op[4 + j] * wp) * inv;
      }
      lnew = mx + __logf(wa + wp);
    }
  }
  acc[0] = r0;
  acc[1] = r1;
  if (o_out) {
    bf16x8 ob;
    for (int j = 0; j < 4; ++j) {
      ob[j] = (bf16)r0[j];
      ob[4 + j] = (bf16)r1[j];
    }
    store_bf16x8(o_out + off, ob);
  }
  if (sub == 0) lse_acc[li] = lnew;
}

hipError_t launch_lse_merge(int64_t n, int32_t H, int32_t D, const void* o_part,
                            const float* lse_part, float* o_acc, float* lse_acc, int32_t first,
                            void* o_out, hipStream_t stream) {
  const int64_t pairs = n * H;
  if (pairs == 0) return hipSuccess;
  const int64_t groups_per_block = 256 / (D / 8);
  const int64_t blocks = (pairs + groups_per_block - 1) / groups_per_block;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const bf16* op = static_cast<const bf16*>(o_part);
  bf16* oo = static_cast<bf16*>(o_out);
  if (D == 128)
    hipLaunchKernelGGL(lse_merge_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, n, H,
                       op, lse_part, o_acc, lse_acc, first, oo);
  else if (D == 64)
    hipLaunchKernelGGL(lse_merge_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, n, H,
                       op, lse_part, o_acc, lse_acc, first, oo);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// All of a ring's step results merged at once: per (row, head), with the
// parts' LSEs l_p and M = max_p l_p, O = sum_p e^(l_p - M) O_p / sum_p
// e^(l_p - M) and LSE = M + log sum_p e^(l_p - M), summed in part order. One
// group of D/8 lanes per (row, head), 16 bytes of each part per lane.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) lse_merge_parts_kernel(
    int64_t n, int32_t H, int32_t parts, const bf16* __restrict__ o_parts,
    const float* __restrict__ lse_parts, bf16* __restrict__ o_out, float* __restrict__ lse_out) {
  constexpr int G = D / 8;
  const int64_t pairs = n * H;
  const int64_t pr = (int64_t)blockIdx.x * (blockDim.x / G) + threadIdx.x / G;
  if (pr >= pairs) return;
  const int sub = threadIdx.x % G;
  const int64_t m = pr / H;
  const int32_t h = (int32_t)(pr - m * H);
  const int64_t li = (int64_t)h * n + m;
  const int64_t off = pr * D + sub * 8;
  const int64_t lstride = (int64_t)H * n, ostride = n * H * D;
  float mx = -INFINITY;
  for (int p = 0; p < parts; ++p) mx = fmaxf(mx, lse_parts[p * lstride + li]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx != -INFINITY) {  // else no part has a key for this row: O = 0, LSE = -inf
    for (int p = 0; p < parts; ++p) {
      const float w = __expf(lse_parts[p * lstride + li] - mx);
      const bf16x8 op = load_bf16x8(o_parts + p * ostride + off);
      wsum += w;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(w, (float)op[j], acc[j]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  bf16x8 ob;
#pragma unroll
  for (int j = 0; j < 8; ++j) ob[j] = (bf16)(acc[j] * inv);
  store_bf16x8(o_out + off, ob);
  if (sub == 0 && lse_out) lse_out[li] = wsum > 0.f ? mx + __logf(wsum) : -INFINITY;
}

hipError_t launch_lse_merge_parts(int64_t n, int32_t H, int32_t D, int32_t parts,
                                  const void* o_parts, const float* lse_parts, void* o_out,
                                  float* lse_out, hipStream_t stream) {
  const int64_t pairs = n * H;
  if (pairs == 0) return hipSuccess;
  const int64_t groups_per_block = 256 / (D / 8);
  const int64_t blocks = (pairs + groups_per_block - 1) / groups_per_block;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const bf16* op = static_cast<const bf16*>(o_parts);
  bf16* oo = static_cast<bf16*>(o_out);
  if (D == 128)
    hipLaunchKernelGGL(lse_merge_parts_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       n, H, parts, op, lse_parts, oo, lse_out);
  else if (D == 64)
    hipLaunchKernelGGL(lse_merge_parts_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       n, H, parts, op, lse_parts, oo, lse_out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Backward preprocess: delta[h, m] = sum_d dO[m,h,d] * O[m,h,d] (fp32).
// One group of D/8 lanes per (row, head); each lane reads 16 bytes of O and dO.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) bwd_prep_kernel(const bf16* __restrict__ o,
                                                       const bf16* __restrict__ d_o,
                                                       const float* __restrict__ lse,
                                                       float* __restrict__ delta,
                                                       int64_t n_local, int32_t H) {
  constexpr int G = D / 8;  // lanes per (row, head)
  const int64_t pairs = n_local * H;
  const int64_t groups_per_grid = (int64_t)gridDim.x * (blockDim.x / G);
  const int sub = threadIdx.x % G;
  for (int64_t pr = (int64_t)blockIdx.x * (blockDim.x / G) + threadIdx.x / G; pr < pairs;
       pr += groups_per_grid) {
    // pr enumerates (m, h) row-major over [n_local, H], matching the memory order
    const int64_t m = pr / H;
    const int32_t h = (int32_t)(pr - m * H);
    const int64_t off = pr * D + sub * 8;
    const bf16x8 ov = load_bf16x8(o + off);
    const bf16x8 dv = load_bf16x8(d_o + off);
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += (float)ov[j] * (float)dv[j];
#pragma unroll
    for (int w = G / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, 64);
    if (sub == 0) {
      const float l = lse[(int64_t)h * n_local + m];
      delta[(int64_t)h * n_local + m] = (l == -INFINITY) ? 0.f : acc;
    }
  }
}

hipError_t launch_bwd_prep(const void* o, const void* d_o, const float* lse, float* delta,
                           int64_t n_local, int32_t H, int32_t D, hipStream_t stream) {
  const int64_t pairs = n_local * H;
  const int per_block = 256 / (D / 8);
  int64_t blocks = (pairs + per_block - 1) / per_block;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) return hipSuccess;
  const bf16* ob = static_cast<const bf16*>(o);
  const bf16* db = static_cast<const bf16*>(d_o);
  if (D == 128)
    hipLaunchKernelGGL(bwd_prep_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, ob, db,
                       lse, delta, n_local, H);
  else if (D == 64)
    hipLaunchKernelGGL(bwd_prep_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, ob, db,
                       lse, delta, n_local, H);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace thdcp
