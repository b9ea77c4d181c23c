// Forward attention of one CP rank's local queries against the full K/V,
// masked by document boundaries and global causal position.
//
// Follows "[PyTorch] Add no-load-balance THD all-gather CP" ("Why": the rank's
// attention steps over the gathered K/V; "Scope and constraints": causal,
// window_size = (-1, 0)) and "[PyTorch] Extend no-load-balance CP to the a2a
// comm type" (body: the mask is the cp_size = 1 mask). Both DUAL_CHUNK_SWAP
// chunks of a document are separate query tiles of this one launch.
//
// gfx950 design: a workgroup of 8 waves owns up to 128 or 256 consecutive
// query rows of one (document piece, head), each wave QB 16-row query blocks:
// QB = 1 (128 rows, ~120 registers, four waves per SIMD) or QB = 2 (256 rows,
// ~180 registers, two per SIMD, each LDS fragment feeding two MFMAs and each
// staged K/V tile serving twice the queries); the plan picks QB = 2 for long
// walks. Keys are walked from the document start in 64-key tiles,
// double-buffered in LDS. Everything is computed in the transposed form
//   S^T = K Q^T  and  O^T = V^T P^T
// with v_mfma_f32_16x16x32_bf16: lane l owns query column l%16 of each block
// and keys 4*(l/16) + i of every 16-key block. K fragments are 16-byte LDS
// reads. V^T fragments are transposing LDS reads (ds_read_b64_tr_b16) of the
// row-major V tile, or, in the transposed-V mode of 256-row tiles at head dim
// 128, 16-byte reads of V^T tiles written by a pre-pass (see kswz_vt). The
// chunk swizzles put the 16 lanes of a group on distinct banks for each read.
// Each fragment is read two MFMA groups ahead of its use (held in place by
// scheduling barriers): the loop was bound by LDS read latency. P feeds the
// second product with no data movement.
//
// The next tile's K/V rows arrive by LDS DMA while the current tile is
// computed: buffer loads that write LDS directly (no staging registers, no
// LDS stores by the waves), whose descriptor ends at the last attended key,
// so rows past it land as zeros with no branch. Padding never enters a
// product.
//
// Online softmax in the log2 domain with lazy rescaling: the running max of a
// query only moves when a tile's scores exceed it by more than kRescaleLog2,
// so probabilities stay below 2^kRescaleLog2 (exact in fp32, representable in
// bf16) and the accumulator rescale, with its cross-lane max, runs only on the
// rare tiles where some lane of the wave crosses that bound (a wave vote). The
// row sum (head dim 128) comes from the matrix core, not from per-element adds:
// one more MFMA per k-step multiplies the same bf16 P by a block of ones, so the
// sum that normalises O is that of the P the P V^T product used (one VALU add
// per score element less; the loop carries more VALU work than its MFMAs hide).
// Only tiles on the causal diagonal apply a per-element mask.
#include "device_common.h"
#include "internal.h"

namespace thdcp {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.f;

// K/V tiles in LDS: BN rows of D bf16 (64 keys; 128 in the transposed-V
// mode), unpadded (LDS DMA writes each wave's 1 KB block contiguously), with
// the 16-byte chunks of row r permuted:
// logical chunk c sits at chunk c ^ kv_swz(r). For D = 128 the swizzle was
// chosen by timing both read patterns of the loop -- the 16-row fragment
// reads (16 rows, one chunk per 16 lanes) and the transposing V^T reads
// (4 rows x 2 chunks per 16 lanes) -- under candidate swizzles on MI355X:
// (r ^ (r >> 2)) & 15 took 1.03 and 1.30 ms where the previous
// (2r + ((r >> 3) & 1)) & 15, which gives 16 lanes distinct chunks as well,
// took 1.95 and 1.57 ms. For D = 64 (two rows per 256-byte bank line) rows
// of one parity take distinct values. Both depend on r mod 16 only: the read
// offsets pass the row within its 16-row group, the DMA the full tile row.
template <int D>
__device__ __forceinline__ int kv_swz(int r) {
  if constexpr (D == 128) {
    const int s = r & 15;
    return s ^ (s >> 2);
  } else {
    return (r >> 1) & 7;
  }
}

// Transposed-V mode (VT: 256-row tiles, D = 128). The transposing LDS reads
// of a row-major V tile cost as much per instruction as a 16-byte read for
// half the bytes (measured on MI355X), so for long walks a pre-pass writes
// V^T (head-dim rows of all keys) and the forward stages V^T tiles: D rows
// of 128 keys (256 bytes), whose A-operand fragments of O^T = V^T P^T are
// plain 16-byte reads of 8 consecutive keys. P^T's k-slots must list those
// same 8 keys, so the S^T row blocks take the K rows in a permuted order:
// row r = 4g + i of key block kb holds key 32(kb>>1) + 8g + 4(kb&1) + i.
// kswz_vt keeps those 16-row K reads free of bank conflicts (it maps the
// rows read by lanes 0..15 of a group onto 16 distinct chunks); V^T tiles
// use kv_swz<128>, as the 16-row reads of a 256-byte-row tile. (vt_swz is
// the swizzle of 64-key V^T tiles: two rows per 256-byte bank line, rows of
// one parity distinct.)
__device__ __forceinline__ int kswz_vt(int r) {
  return (r & 3) | (((r >> 3) & 1) << 2) | (((r >> 4) & 1) << 3);
}
__device__ __forceinline__ int vt_swz(int r) { return (r >> 1) & 7; }

template <int D, int BN>
struct FwdSmem {
  static constexpr int ROWB = D * 2;            // bytes per row
  static constexpr int TILEB = BN * ROWB;       // bytes per K or V tile
  __attribute__((aligned(1024))) char k[2][TILEB];
  __attribute__((aligned(1024))) char v[2][TILEB];
};

// Eight waves per workgroup; QB 16-row query blocks per wave, so a tile holds
// 128 * QB rows.
constexpr int kFwdThreads = 512;

// K/V row of key j: j - kv_sub (global order, or one rank's block of it
// under NO_LOAD_BALANCE), or, when MAPPED, kv_row[j] - kv_sub (rank-major
// K/V, or one rank's block of it: the restore fused into the loads).
// BAND: a general key band [g - wl, g + wr]; otherwise the causal mask
// (wl unbounded, wr = 0, folded at compile time).
// VT: V is read as V^T tiles of vt (head h's D rows of vt_pitch keys, keys in
// global order) instead of V rows. The second bound is waves per SIMD: two
// workgroups per CU with QB = 1, one with QB = 2, which caps the registers
// at 512 / that.
template <int D, int QB, bool MAPPED, bool BAND, bool VT>
__global__ void __launch_bounds__(kFwdThreads, QB == 2 ? 2 : 4)
attn_fwd_kernel(const FwdTile* __restrict__ tiles, int32_t H, const bf16* __restrict__ q,
                const bf16* __restrict__ k, const bf16* __restrict__ v,
                const int32_t* __restrict__ kv_row, int32_t kv_sub, uint32_t kv_bytes,
                int32_t wl_arg, int32_t wr_arg, bf16* __restrict__ o, float* __restrict__ lse,
                int64_t n_local, float scale_log2, SplitWs split, const bf16* __restrict__ vt,
                int32_t vt_pitch) {
  static_assert(!VT || (D == 128 && QB == 2), "transposed V: 256-row tiles of head dim 128");
  constexpr int kThreads = kFwdThreads;
  // Keys per tile: 128 with transposed V (one workgroup per CU, 128 KB of
  // LDS for two K and two V^T tiles), else 64.
  constexpr int BN = VT ? 2 * kFwdBN : kFwdBN;
  constexpr int KS = D / 32;   // 16x16x32 k-steps over the head dim
  constexpr int NB = D / 16;   // 16-wide blocks of the head dim
  constexpr int KB = BN / 16;  // 16-key blocks per tile
  constexpr int kPf = 2;       // LDS fragment reads in flight ahead of their MFMAs
  constexpr int ROWB = FwdSmem<D, BN>::ROWB;
  constexpr int TILEB = FwdSmem<D, BN>::TILEB;
  constexpr int LPR = ROWB / 16;               // lanes (16-byte chunks) per row
  constexpr int RPI = 1024 / ROWB;             // rows per wave DMA instruction
  constexpr int NI = TILEB / 1024 / (kThreads / 64);  // DMA instructions per wave per tensor
  static_assert(NI * (kThreads / 64) * 1024 == TILEB, "tile splits evenly over the waves");
  __shared__ FwdSmem<D, BN> sm;

  const int tile_id = blockIdx.x / H;
  const int h = blockIdx.x - tile_id * H;
  const FwdTile t = tiles[tile_id];
  // Wave index, made wave-uniform explicitly so it and the LDS addresses
  // derived from it live in scalar registers.
  const int w = wave_uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;  // query column of this lane (and row of A operands)
  const int G = lane >> 4;    // 16-lane group
  const int64_t rs = (int64_t)H * D;
  const int64_t head_off = (int64_t)h * D;
  const int wl = BAND ? wl_arg : kUnbounded;
  const int wr = BAND ? wr_arg : 0;

  // Query rows of this lane: block qb holds tile row (w*QB + qb)*16 + l16.
  // Key j is allowed iff my_lo <= j <= my_hi (and j is below the tile range's
  // end); padding rows have my_hi = -1 and allow nothing.
  int my_g[QB], my_lo[QB], my_hi[QB];
  bool in_tile[QB];
  int64_t m_row[QB];
  bf16x8 qf[QB][KS];  // B operand of S^T: query l16, head dims kk*32 + G*8 .. +7
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = (w * QB + qb) * 16 + l16;
    in_tile[qb] = r < t.n;
    const int g = t.g0 + r;
    const bool valid = in_tile[qb] && g < t.e;
    m_row[qb] = (int64_t)t.m0 + r;
    my_g[qb] = valid ? g : -1;
    my_lo[qb] = g - wl;
    my_hi[qb] = valid ? g + wr : -1;
    const bf16* qp = q + m_row[qb] * rs + head_off + G * 8;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      qf[qb][kk] = valid ? load_bf16x8(qp + kk * 32) : zero_bf16x8();
  }

  f32x4 oacc[QB][NB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[qb][nb][i] = 0.f;
  float m_run[QB], l_part[QB];  // running max (log2 units); this lane's share of the row sum
  // Head dim 128: row sums on the matrix core, lsum[qb] += 1 P^T per k-step
  // (all four entries hold the sum of the lane's query; measured on one
  // 75600-token document: forward -2.4..-3.9% against per-element fp32 adds).
  // Head dim 64 keeps the per-lane fp32 adds: there the eight more registers
  // cost the 128-row instance a workgroup per CU (nlb_32k at head dim 64: +10%).
  constexpr bool kMfmaRowSum = D == 128;
  f32x4 lsum[QB];
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (bf16)1.f;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_part[qb] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) lsum[qb][i] = 0.f;
  }

  // Staging by LDS DMA: DMA instruction j of wave w fills rows
  // [(w*NI + j)*RPI, +RPI) of the tile; lane i loads row (w*NI + j)*RPI +
  // i/LPR, physical chunk i%LPR, i.e. logical chunk (i%LPR) ^ kv_swz(row).
  // No registers hold the tile and nothing is written to LDS by the waves;
  // the data lands asynchronously (counted by vmcnt).
  const uint32_t row_bytes = (uint32_t)(rs * 2);
  int drow[NI];
  uint32_t dcol[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    drow[j] = (w * NI + j) * RPI + lane / LPR;
    dcol[j] = (uint32_t)(((lane % LPR) ^ (VT ? kswz_vt(drow[j]) : kv_swz<D>(drow[j]))) * 16);
  }
  // V^T staging (VT): a V^T row is BN keys (256 bytes with 128-key tiles, 16
  // chunks). DMA instruction j of wave w fills rows (head dims)
  // [(w*NI + j)*VRPI, +VRPI): lane i loads dim (w*NI + j)*VRPI + i/VLPR,
  // physical chunk i%VLPR, i.e. keys k0 + 8*((i%VLPR) ^ vtswz(dim)) .. +7.
  // The pitch leaves 128 keys past the last tile start, and keys no local
  // query attends (padding among them) hold 0 in vt, so the keys of a tile
  // past its range end enter P V^T as 0 * finite.
  constexpr int VLPR = BN * 2 / 16;      // lanes (16-byte chunks) per V^T row
  constexpr int VRPI = 64 / VLPR;        // V^T rows per DMA instruction
  auto vtswz = [&](int r) { return BN == 128 ? kv_swz<128>(r) : vt_swz(r); };
  uint32_t vtoff[NI];
  if constexpr (VT) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int dr = (w * NI + j) * VRPI + lane / VLPR;
      vtoff[j] = (uint32_t)dr * (uint32_t)vt_pitch * 2u +
                 (uint32_t)(((lane % VLPR) ^ vtswz(dr)) * 16);
    }
  }
  auto load_vt = [&](int k0, char* dst) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(vt + (int64_t)h * D * vt_pitch + k0,
                                               (uint32_t)(((int64_t)D * vt_pitch - k0) * 2));
#pragma unroll
    for (int j = 0; j < NI; ++j) dma16(r, vtoff[j], dst + (w * NI + j) * 1024);
  };
  // Rows [k0, k0 + BN) of K or V into LDS tile dst, for a tile of a key range
  // ending at kend; a row at or past kend reads 0 with no branch.
  //  - Unmapped: the descriptor runs from row k0 - kv_sub to the range end,
  //    so offsets of rows past it land past its end.
  //  - MAPPED: pos[] holds this lane's rows of the tile, looked up one tile
  //    ahead of the loads that use them so the lookup's latency stays off the
  //    prefetch path; a skipped row gets an offset past the descriptor, which
  //    spans all kv rows (below 2 GiB, checked on the host).
  auto rows_pos = [&](int k0, int kend, int (&pos)[NI]) {
    if constexpr (MAPPED) {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int key = k0 + drow[j];
        const int r = kv_row[min(key, kend - 1)] - kv_sub;
        pos[j] = key < kend ? r : -1;
      }
    }
  };
  auto load_rows = [&](const bf16* x, int k0, int kend, const int (&pos)[NI], char* dst) {
    if constexpr (MAPPED) {
      const __amdgpu_buffer_rsrc_t r = make_rsrc(x + head_off, kv_bytes);
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const uint32_t off = pos[j] >= 0 ? (uint32_t)pos[j] * row_bytes + dcol[j] : 0xFFFFFFF0u;
        dma16(r, off, dst + (w * NI + j) * 1024);
      }
    } else {
      const int64_t n = (int64_t)kend - k0;
      const __amdgpu_buffer_rsrc_t r =
          n > 0 ? make_rsrc(x + (int64_t)(k0 - kv_sub) * rs + head_off, (uint32_t)(n * rs * 2))
                : make_rsrc(x, 0u);
#pragma unroll
      for (int j = 0; j < NI; ++j)
        dma16(r, (uint32_t)drow[j] * row_bytes + dcol[j], dst + (w * NI + j) * 1024);
    }
  };
  // LDS byte offsets of this lane's fragment reads (lane constants): the K
  // fragment of k-step kk and key block kb is row kb*16 + l16, logical chunk
  // kk*4 + G; the V^T reads of head-dim block nb are rows 32ks + 4G +
  // (l16 >> 2) (+16), logical chunk 2nb + ((l16 & 3) >> 1), half l16 & 1.
  const int ksw = G ^ kv_swz<D>(l16);
  const int vr = G * 4 + (l16 >> 2);
  const int vsw = ((l16 >> 1) & 1) ^ kv_swz<D>(vr);
  auto k_off = [&](int kb, int kk) {
    if constexpr (VT)  // row 32(kb>>1) + 8(l16>>2) + 4(kb&1) + (l16&3), whose kswz_vt is l16
      return (32 * (kb >> 1) + 8 * (l16 >> 2) + 4 * (kb & 1) + (l16 & 3)) * ROWB +
             (((kk * 4 + G) ^ l16) << 4);
    return (kb * 16 + l16) * ROWB + (((kk * 4) ^ ksw) << 4);
  };
  auto v_off = [&](int ks, int half, int nb) {
    return (32 * ks + 16 * half + vr) * ROWB + (((2 * nb) ^ vsw) << 4) + 8 * (l16 & 1);
  };
  // S^T = K Q^T for the K tile in LDS buffer kbuf: each K fragment (one
  // 16-byte LDS read) feeds the MFMAs of all QB query blocks.
  auto scores = [&](int kbuf, f32x4 (&s)[QB][KB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[qb][kb][i] = 0.f;
    // KS * KB fragment reads, each feeding QB MFMAs, read kPf ahead into a
    // ring; the scheduling barriers keep the compiler from sinking the reads
    // back next to their MFMAs.
    constexpr int kN = KS * KB;
    bf16x8 ring[kPf + 1];
    auto fetch = [&](int n) {
      ring[n % (kPf + 1)] =
          load_bf16x8(reinterpret_cast<const bf16*>(&sm.k[kbuf][k_off(n % KB, n / KB)]));
    };
#pragma unroll
    for (int n = 0; n < kPf; ++n) fetch(n);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      if (n + kPf < kN) fetch(n + kPf);
      const int kb = n % KB, kk = n / KB;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma16(ring[n % (kPf + 1)], qf[qb][kk], s[qb][kb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Band / padding mask: key j is allowed iff my_lo <= j <= my_hi and
  // j < kend (the end of the key range the tile belongs to).
  auto mask = [&](int k0, int kend, f32x4 (&s)[QB][KB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = VT ? k0 + 32 * (kb >> 1) + 8 * G + 4 * (kb & 1) + i
                             : k0 + kb * 16 + G * 4 + i;
          bool out = key > my_hi[qb] || key >= kend;
          if constexpr (BAND) out = out || key < my_lo[qb];
          if (out) s[qb][kb][i] = -INFINITY;
        }
  };
  // Lazy rescale: the running max of a query moves only when some score of
  // the tile exceeds it by more than kRescaleLog2 (decided by a wave vote, so
  // the cross-lane max and the accumulator rescale run only on such tiles).
  auto softmax_max = [&](f32x4 (&s)[QB][KB]) {
    float lm[QB];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = s[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[qb][kb][i]);
      lm[qb] = mx * scale_log2;
      need |= lm[qb] > m_run[qb] + kRescaleLog2;
    }
    if (__any(need)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float rm = group_max4(lm[qb]);  // the row's tile max (uniform per query)
        const float m_new = rm > m_run[qb] + kRescaleLog2 ? rm : m_run[qb];
        const float alpha = m_new == m_run[qb] ? 1.f : fast_exp2(m_run[qb] - m_new);
        m_run[qb] = m_new;
        if constexpr (kMfmaRowSum) {
#pragma unroll
          for (int i = 0; i < 4; ++i) lsum[qb][i] *= alpha;
        } else {
          l_part[qb] *= alpha;
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[qb][nb][i] *= alpha;
      }
    }
  };
  // P = exp2(S*scale - m) and O^T += V^T P^T. k-step ks covers key blocks
  // 2ks, 2ks+1: slot j of this lane is key (2ks + j/4)*16 + 4*G + j%4 --
  // accumulator entries of s[.][2ks], s[.][2ks+1]. The V^T operand (lane =
  // head dim, slots = those keys) is a plain read of the V^T tile (VT) or two
  // transposing reads of the row-major V tile, shared by all query blocks.
  // The next k-step's exponentials are spread over this k-step's MFMA steps
  // (the scheduling barriers keep the compiler from moving them there on its
  // own): forward -1.3% on one 75600-token document, bit-identical.
  auto softmax_pv = [&](int vbuf, f32x4 (&s)[QB][KB]) {
    float m_use[QB], ps[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m_use[qb] = m_run[qb] == -INFINITY ? 0.f : m_run[qb];
      ps[qb] = 0.f;
    }
    // Exponential e of k-step ks: query block e / 8, key block 2ks + (e % 8) / 4,
    // entry e % 4 (each block's sum in the order of a plain loop).
    auto expo = [&](int ks, int e) {
      const int qb = e / 8, kb = 2 * ks + (e % 8) / 4, i = e % 4;
      const float p = fast_exp2(fmaf(s[qb][kb][i], scale_log2, -m_use[qb]));
      s[qb][kb][i] = p;
      if constexpr (!kMfmaRowSum) ps[qb] += p;
    };
    constexpr int kE = QB * 8;       // exponentials per k-step
    constexpr int kEPer = kE / NB;   // of the next k-step per P V^T step
    static_assert(kE % NB == 0, "exponentials split evenly over the P V^T steps");
#pragma unroll
    for (int e = 0; e < kE; ++e) expo(0, e);
#pragma unroll
    for (int ks = 0; ks < KB / 2; ++ks) {
      bf16x8 pb[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if constexpr (!kMfmaRowSum) {
          l_part[qb] += ps[qb];
          ps[qb] = 0.f;
        }
        pb[qb] = pack8(s[qb][2 * ks], s[qb][2 * ks + 1]);
      }
      bf16x8 ring[kPf + 1];
      auto fetch = [&](int nb) {
        if constexpr (VT)  // V^T row nb*16 + l16, keys 32ks + 8G .. +7
          ring[nb % (kPf + 1)] = load_bf16x8(reinterpret_cast<const bf16*>(
              &sm.v[vbuf][(nb * 16 + l16) * (BN * 2) +
                          (((ks * 4 + G) ^ vtswz(nb * 16 + l16)) << 4)]));
        else
          ring[nb % (kPf + 1)] =
              concat4(lds_read_tr4(reinterpret_cast<const bf16*>(&sm.v[vbuf][v_off(ks, 0, nb)])),
                      lds_read_tr4(reinterpret_cast<const bf16*>(&sm.v[vbuf][v_off(ks, 1, nb)])));
      };
#pragma unroll
      for (int nb = 0; nb < kPf; ++nb) fetch(nb);
      __builtin_amdgcn_sched_barrier(0);
      // The next k-step's exponentials, kEPer beside each step's MFMAs.
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (nb + kPf < NB) fetch(nb + kPf);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[qb][nb] = mfma16(ring[nb % (kPf + 1)], pb[qb], oacc[qb][nb]);
        if (kMfmaRowSum && nb == 0) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) lsum[qb] = mfma16(ones, pb[qb], lsum[qb]);
        }
        if (ks + 1 < KB / 2) {
#pragma unroll
          for (int e = nb * kEPer; e < (nb + 1) * kEPer; ++e) expo(ks + 1, e);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Key tiles: those of [ks0, ke0), then those of [ks1, ke1).
  const int nt0 = t.ke0 > t.ks0 ? (t.ke0 - t.ks0 + BN - 1) / BN : 0;
  const int nt1 = t.ke1 > t.ks1 ? (t.ke1 - t.ks1 + BN - 1) / BN : 0;
  const int ntiles = nt0 + nt1;
  auto tile_k0 = [&](int it) { return it < nt0 ? t.ks0 + it * BN : t.ks1 + (it - nt0) * BN; };
  auto tile_kend = [&](int it) { return it < nt0 ? t.ke0 : t.ke1; };

  // Double-buffered K/V tiles: the next tile's loads are issued before the
  // current tile's MFMAs and written to LDS after them; one barrier per tile.
  // Waves whose rows cannot see a tile skip it (scalar branch).
  const int row0 = w * QB * 16;
  const bool wave_has_rows = (row0 < t.n) && (t.g0 + row0 < t.e);
  const int wrow_last = min(row0 + QB * 16 - 1, t.n - 1);
  // Keys the wave's rows can reach: [wave_kmin, wave_kmax]; a tile needs the
  // per-element mask unless every key of it is inside every row's band.
  const int wave_kmax =
      wave_uniform(wave_has_rows ? min(t.g0 + wrow_last + wr, t.e - 1) : -1);
  const int wave_kmin = wave_uniform(t.g0 + row0 - wl);
  const int wave_gmin = wave_uniform(t.g0 + row0);
  const int wave_gmax = wave_uniform(t.g0 + row0 + QB * 16 - 1);
  const bool wave_all_valid =
      wave_uniform((row0 + QB * 16 - 1 < t.n) && (t.g0 + row0 + QB * 16 - 1 < t.e)) != 0;
  // The second tile's rows are looked up beside the first's, so the prologue
  // waits on one row-map round trip before the first K/V loads, not two.
  int pos[NI], pos1[NI] = {};
  if (ntiles > 0) {
    rows_pos(tile_k0(0), tile_kend(0), pos);
    if (ntiles > 1) rows_pos(tile_k0(1), tile_kend(1), pos1);
    load_rows(k, tile_k0(0), tile_kend(0), pos, sm.k[0]);
    if constexpr (VT) load_vt(tile_k0(0), sm.v[0]);
    else load_rows(v, tile_k0(0), tile_kend(0), pos, sm.v[0]);
#pragma unroll
    for (int j = 0; j < NI; ++j) pos[j] = pos1[j];
  }
  wait_vmem();
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int k0 = tile_k0(it);
    const int kend = tile_kend(it);
    const int cur = it & 1;
    const bool has_next = it + 1 < ntiles;
    if (has_next) {  // in flight during this tile's compute (the other buffer's
                     // last readers passed the previous barrier)
      load_rows(k, tile_k0(it + 1), tile_kend(it + 1), pos, sm.k[cur ^ 1]);
      if constexpr (VT) load_vt(tile_k0(it + 1), sm.v[cur ^ 1]);
      else load_rows(v, tile_k0(it + 1), tile_kend(it + 1), pos, sm.v[cur ^ 1]);
      if (it + 2 < ntiles) rows_pos(tile_k0(it + 2), tile_kend(it + 2), pos);
    }
    if (k0 <= wave_kmax && (!BAND || k0 + BN - 1 >= wave_kmin)) {
      f32x4 s[QB][KB];
      scores(cur, s);
      if (!wave_all_valid || k0 + BN - 1 > wave_gmin + wr || (BAND && k0 < wave_gmax - wl) ||
          k0 + BN > kend)
        mask(k0, kend, s);
      softmax_max(s);
      softmax_pv(cur, s);
    }
    wait_vmem();  // this wave's DMA of the next tile has landed
    __syncthreads();
  }

  // The row sum as four shares, one per lane group, as the merge and the
  // epilogue take it.
  if constexpr (kMfmaRowSum) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_part[qb] = G == 0 ? lsum[qb][0] : 0.f;
  }

  if (t.nparts > 1) {
    // Split key walk: this part's state (accumulators, then per query block
    // the running max and this lane's row-sum share) goes to its scratch slot
    // in lane order; the last part to finish rescales every part's state to
    // the largest running max and sums them in part order, which is the
    // online softmax's own merge of two key ranges.
    constexpr int NBLK = kThreads / 64 * QB;  // 16-row query blocks per tile
    auto acc_at = [&](int x, int b, int nb) {
      return reinterpret_cast<f32x4*>(split_slot<D, NBLK * 16>(split.part, x, h, H)) +
             ((b * NB + nb) * 64 + lane);
    };
    auto st_at = [&](int x, int b) {
      return reinterpret_cast<float2*>(split_slot<D, NBLK * 16>(split.part, x, h, H) +
                                       NBLK * NB * 256) +
             (b * 64 + lane);
    };
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int b = w * QB + qb;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) *acc_at(t.slot + t.part, b, nb) = oacc[qb][nb];
      *st_at(t.slot + t.part, b) = make_float2(m_run[qb], l_part[qb]);
    }
    if (!split_arrive(split.cnt + (int64_t)t.group * H + h, t.nparts)) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int b = w * QB + qb;
      float mx = -INFINITY;
      for (int p = 0; p < t.nparts; ++p) mx = fmaxf(mx, st_at(t.slot + p, b)->x);
      l_part[qb] = 0.f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[qb][nb][i] = 0.f;
      for (int p = 0; p < t.nparts; ++p) {
        const float2 st = *st_at(t.slot + p, b);
        const float f = st.x == -INFINITY ? 0.f : fast_exp2(st.x - mx);
        l_part[qb] = fmaf(st.y, f, l_part[qb]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const f32x4 a = *acc_at(t.slot + p, b, nb);
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[qb][nb][i] = fmaf(a[i], f, oacc[qb][nb][i]);
        }
      }
      m_run[qb] = mx;
    }
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = group_sum4(l_part[qb]);
    if (!in_tile[qb]) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    bf16* op = o + m_row[qb] * rs + head_off;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // accumulator rows (head dims) nb*16 + 4*G + 0..3 of query l16
      bf16x4 out;
#pragma unroll
      for (int j = 0; j < 4; ++j) out[j] = (bf16)(oacc[qb][nb][j] * inv);
      store_bf16x4(op + nb * 16 + G * 4, out);
    }
    if (G == 0) {
      lse[(int64_t)h * n_local + m_row[qb]] =
          (my_g[qb] >= 0 && l > 0.f) ? (m_run[qb] + __log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

// Tiles of 128 rows (QB = 1: waves of 16 rows, four per SIMD) or 256 (QB = 2:
// waves of 32 rows, two per SIMD, one workgroup per CU, every K and V^T
// fragment read from LDS feeding two MFMAs and every staged K/V tile serving
// 256 queries). The plan picks 256-row tiles for shares whose average walk is
// long (measured on MI355X: one 75600-token document 6.9-7.0 against 7.3-7.4
// ms with 128-row tiles of 32-row waves) and 128 otherwise (the
// multi-document shares' short tiles: 10-15% faster).
template <int D, int QB, bool VT>
hipError_t launch_fwd_d(const FwdTile* tiles, int64_t blocks, int32_t H, const bf16* q,
                        const bf16* k, const bf16* v, const int32_t* kv_row, int32_t kv_sub,
                        uint32_t kv_bytes, Band band, bf16* o, float* lse, int64_t n_local,
                        float scale_log2, SplitWs split, const bf16* vt, int32_t vt_pitch,
                        hipStream_t stream) {
#define THDCP_FWD(MM, BB)                                                                   \
  hipLaunchKernelGGL((attn_fwd_kernel<D, QB, MM, BB, VT>), dim3((unsigned)blocks),           \
                     dim3(kFwdThreads), 0, stream, tiles, H, q, k, v, kv_row, kv_sub,        \
                     kv_bytes, band.wl, band.wr, o, lse, n_local, scale_log2, split, vt,     \
                     vt_pitch)
  if (kv_row && band.causal)
    THDCP_FWD(true, false);
  else if (kv_row)
    THDCP_FWD(true, true);
  else if (band.causal)
    THDCP_FWD(false, false);
  else
    THDCP_FWD(false, true);
#undef THDCP_FWD
  return hipGetLastError();
}

// V^T for the transposed-V forward: vt[(h*128 + d) * pitch + j] = V of key j
// (K/V row j - sub, or kv_row[j] - sub), head h, dim d, for j < T; 0 for
// j >= T and for keys in the zero ranges (keys no local query attends:
// padding and other documents). One workgroup per 64 keys and head: the rows
// are read as 16-byte chunks into LDS and written back as 8-key chunks of
// one dim.
__global__ void __launch_bounds__(256)
v_transpose_kernel(const bf16* __restrict__ v, const int32_t* __restrict__ kv_row, int32_t sub,
                   int32_t T, int32_t H, const ZeroRange* __restrict__ zr, int32_t n_zr,
                   bf16* __restrict__ vt, int32_t pitch) {
  constexpr int D = 128;
  __shared__ bf16 tile[64][D + 8];
  const int k0 = blockIdx.x * 64;
  const int h = blockIdx.y;
  const int64_t rs = (int64_t)H * D;
  for (int c = threadIdx.x; c < 64 * (D / 8); c += 256) {
    const int r = c / (D / 8), ch = c % (D / 8);
    const int key = k0 + r;
    bool live = key < T;
    if (live && n_zr > 0) {  // last zero range starting at or before key
      int lo = 0, hi = n_zr - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (zr[mid].r0 <= key) lo = mid; else hi = mid - 1;
      }
      live = !(zr[lo].r0 <= key && key < zr[lo].r1);
    }
    bf16x8 x = zero_bf16x8();
    if (live) {
      const int64_t row = (int64_t)(kv_row ? kv_row[key] : key) - sub;
      x = load_bf16x8(v + row * rs + (int64_t)h * D + ch * 8);
    }
    store_bf16x8(&tile[r][ch * 8], x);
  }
  __syncthreads();
  for (int c = threadIdx.x; c < D * 8; c += 256) {
    const int d = c / 8, kc = c % 8;
    bf16x8 y;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = tile[kc * 8 + e][d];
    store_bf16x8(vt + ((int64_t)h * D + d) * pitch + k0 + kc * 8, y);
  }
}

}  // namespace

int32_t vt_pitch_for(int64_t T) { return (int32_t)((T + 63) / 64 * 64 + 128); }

hipError_t launch_v_transpose(const void* v, KvRows kv, int32_t H, int32_t D,
                              const ZeroRange* zr, int32_t n_zr, void* vt, int32_t pitch,
                              hipStream_t stream) {
  if (D != 128 || pitch < vt_pitch_for(kv.rows) || pitch % 64 != 0)
    return hipErrorInvalidValue;
  if (H == 0 || kv.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(v_transpose_kernel, dim3((unsigned)(pitch / 64), (unsigned)H), dim3(256), 0,
                     stream, static_cast<const bf16*>(v), kv.map, (int32_t)kv.sub,
                     (int32_t)kv.rows, H, zr, n_zr, static_cast<bf16*>(vt), pitch);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const FwdTile* tiles, int32_t n_tiles, int32_t H, int32_t D,
                           int32_t rows, const void* q, const void* k, const void* v, KvRows kv,
                           Band band, void* o, float* lse, int64_t n_local, float scale,
                           SplitWs split, const void* vt, int32_t vt_pitch,
                           hipStream_t stream) {
  const int64_t blocks = (int64_t)n_tiles * H;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const float scale_log2 = scale * kLog2e;
  const bf16* qp = static_cast<const bf16*>(q);
  const bf16* kb = static_cast<const bf16*>(k);
  const bf16* vb = static_cast<const bf16*>(v);
  const bf16* vtb = static_cast<const bf16*>(vt);
  bf16* ob = static_cast<bf16*>(o);
  const int64_t kv_bytes = kv.rows * H * D * 2;
  if (kv.map && kv_bytes >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const uint32_t kvb = kv.map ? (uint32_t)kv_bytes : 0u;
  if (vt && (D != 128 || rows != kFwdBMLong || (int64_t)D * vt_pitch * 2 >= ((int64_t)1 << 31)))
    return hipErrorInvalidValue;
#define THDCP_FWD_D(DD, QQ, VV)                                                              \
  return launch_fwd_d<DD, QQ, VV>(tiles, blocks, H, qp, kb, vb, kv.map, (int32_t)kv.sub, kvb, \
                                  band, ob, lse, n_local, scale_log2, split, vtb, vt_pitch,   \
                                  stream)
  if (D == 128 && rows == kFwdBMLong && vt) THDCP_FWD_D(128, 2, true);
  if (D == 128 && rows == kFwdBMLong) THDCP_FWD_D(128, 2, false);
  if (D == 128 && rows == kFwdBM) THDCP_FWD_D(128, 1, false);
  if (D == 64 && rows == kFwdBMLong) THDCP_FWD_D(64, 2, false);
  if (D == 64 && rows == kFwdBM) THDCP_FWD_D(64, 1, false);
#undef THDCP_FWD_D
  return hipErrorInvalidValue;
}

}  // namespace thdcp
