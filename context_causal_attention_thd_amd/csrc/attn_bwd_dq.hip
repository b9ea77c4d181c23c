// Backward, query side: dQ for the local rows of one CP rank's share
// ("[PyTorch] Add no-load-balance THD all-gather CP", sequence diagram: the
// backward of the rank's attention steps). Each query row's gradient only
// needs that row's LSE and delta, so dQ is computed query-tile-major, exactly
// like the forward pass: no atomics, every local row written once (padding
// rows 0), bit-identical from run to run.
//
// gfx950 design (mirrors the forward kernel): a workgroup of 4 or 8 waves owns
// up to 128 or 256 consecutive query rows of one (document piece, head), 32
// per wave (8 waves, one workgroup per CU, for the plans with long walks:
// each staged K/V tile serves twice the queries), and walks the keys from the
// document start in 64-key tiles, double-buffered in LDS; the next tile
// arrives by LDS DMA (buffer loads that write LDS directly, no registers)
// while the current one is computed. Per tile, with
// v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T, dP^T = V dO^T   (A = K / V rows from LDS, B = Q / dO regs)
//   P^T = exp(S^T - LSE), dS^T = P^T (dP^T - delta)   (lane-local per query)
//   dQ^T += K^T dS^T             (A = K^T by transposing LDS reads)
// dS^T leaves the first products in exactly the B-operand layout of the
// third, so it never touches LDS. Every LDS operand is read two MFMAs ahead
// of its use (held in place by scheduling barriers), so an MFMA does not wait
// on a read issued just before it: the loop was bound by LDS read latency
// (without the reads it ran 1.8x faster).
#include "device_common.h"
#include "internal.h"

namespace thdcp {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// K/V tiles in LDS: kFwdBN rows of D bf16, unpadded (LDS DMA writes each
// wave's 1 KB block contiguously), with the 16-byte chunks of row r permuted:
// logical chunk c sits at chunk c ^ dq_swz(r). For D = 128 the swizzle maps
// every 16 consecutive rows one to one onto 0..15 (the 32-row K and V
// fragment reads: 16 rows of one chunk per 16 lanes) and gives rows
// 4i..4i+3 distinct multiples of 4 (the transposing K^T reads: 4 rows of 4
// adjacent chunks per 32 lanes), so both read patterns are free of bank
// conflicts. For D = 64 (two rows per 256-byte bank line) rows of one parity
// take distinct values.
template <int D>
__device__ __forceinline__ int dq_swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (r >> 1) & 7;
}

template <int D>
struct DqSmem {
  static constexpr int ROWB = D * 2;            // bytes per row
  static constexpr int TILEB = kFwdBN * ROWB;   // bytes per K or V tile
  __attribute__((aligned(1024))) char k[2][TILEB];
  __attribute__((aligned(1024))) char v[2][TILEB];
};

// K/V row of key j: j - kv_sub (global order, or one rank's block of it
// under NO_LOAD_BALANCE), or, when MAPPED, kv_row[j] - kv_sub (rank-major
// K/V, or one rank's block of it: the restore fused into the loads).
// DELTA: compute delta = rowsum(dO * O) for the tile's rows here (from the
// dO fragments already loaded and the matching O fragments) and write it for
// the dK/dV kernel, instead of reading it from a separate preprocess launch.
// BAND: a general key band [g - wl, g + wr]; otherwise the causal mask
// (wl unbounded, wr = 0, folded at compile time).
// WAVES: 4 (128-row tiles) or 8 (256-row tiles); two waves per SIMD either way.
template <int D, int WAVES, bool MAPPED, bool DELTA, bool BAND>
__global__ void __launch_bounds__(WAVES * 64, 2)
attn_bwd_dq_kernel(const FwdTile* __restrict__ tiles, int32_t H, const bf16* __restrict__ q,
                   const bf16* __restrict__ k, const bf16* __restrict__ v,
                   const int32_t* __restrict__ kv_row, int32_t kv_sub, uint32_t kv_bytes,
                   int32_t wl_arg, int32_t wr_arg, const bf16* __restrict__ d_o,
                   const bf16* __restrict__ o,
                   const float* __restrict__ lse, float* __restrict__ delta,
                   float* __restrict__ dq, int64_t n_local, int32_t accumulate,
                   float scale, float scale_log2, int32_t n_attn_blocks, SplitWs split,
                   DqExtras ex) {
  constexpr int kThreads = WAVES * 64;
  constexpr int BN = kFwdBN;
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int ROWB = DqSmem<D>::ROWB;
  constexpr int TILEB = DqSmem<D>::TILEB;
  constexpr int LPR = ROWB / 16;                       // lanes (16-byte chunks) per row
  constexpr int RPI = 1024 / ROWB;                     // rows per wave DMA instruction
  constexpr int NI = TILEB / 1024 / WAVES;             // DMA instructions per wave per tensor
  static_assert(NI * WAVES * 1024 == TILEB, "tile splits evenly over the waves");
  __shared__ DqSmem<D> sm;

  if ((int)blockIdx.x >= n_attn_blocks) {  // gated zeroing workgroups
    zero_untouched_block(blockIdx.x - n_attn_blocks, ex.zr, ex.n_zr, ex.zero_rows, kv_row, kv_sub,
                         (int64_t)H * D, ex.dk, ex.dv);
    return;
  }
  const int tile_id = blockIdx.x / H;
  const int h = blockIdx.x - tile_id * H;
  const FwdTile t = tiles[tile_id];
  // Wave index, made wave-uniform explicitly so it and the LDS addresses
  // derived from it live in scalar registers.
  const int w = wave_uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int li = lane & 31;
  const int hh = lane >> 5;
  const int64_t rs = (int64_t)H * D;
  const int64_t head_off = (int64_t)h * D;

  const int r = w * 32 + li;
  const bool in_tile = r < t.n;
  const int g = t.g0 + r;
  const bool valid = in_tile && g < t.e;
  const int64_t m = (int64_t)t.m0 + r;
  // Key j is allowed iff my_lo <= j <= my_hi (and below the tile range's
  // end); padding rows allow nothing.
  const int wl = BAND ? wl_arg : kUnbounded;
  const int wr = BAND ? wr_arg : 0;
  const int my_lo = g - wl;
  const int my_hi = valid ? g + wr : -1;

  // Q and dO fragments (B operands): query li, head dims kk*16 + hh*8 .. +7
  bf16x8 qf[KSTEPS], dof[KSTEPS];
  {
    const int64_t off = m * rs + head_off + hh * 8;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      qf[kk] = valid ? load_bf16x8(q + off + kk * 16) : zero_bf16x8();
      dof[kk] = valid ? load_bf16x8(d_o + off + kk * 16) : zero_bf16x8();
    }
  }
  const float lse2 = valid ? lse[(int64_t)h * n_local + m] * kLog2e : 0.f;
  float dlt;
  if constexpr (DELTA) {
    // This lane holds head dims kk*16 + hh*8 .. +7 of its row's dO; the two
    // halves of the wave hold the two halves of the row.
    const int64_t off = m * rs + head_off + hh * 8;
    float part = 0.f;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const bf16x8 of = valid ? load_bf16x8(o + off + kk * 16) : zero_bf16x8();
#pragma unroll
      for (int j = 0; j < 8; ++j) part = fmaf((float)dof[kk][j], (float)of[j], part);
    }
    dlt = part + __shfl_xor(part, 32, 64);  // 0 on padding rows (dO taken as 0)
    if (hh == 0 && in_tile && t.part == 0) delta[(int64_t)h * n_local + m] = dlt;
  } else {
    dlt = valid ? delta[(int64_t)h * n_local + m] : 0.f;
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  const int wrow_last = min(w * 32 + 31, t.n - 1);
  const bool wave_has_rows = (w * 32 < t.n) && (t.g0 + w * 32 < t.e);
  // Keys the wave's rows can reach: [wave_kmin, wave_kmax].
  const int wave_kmax =
      wave_uniform(wave_has_rows ? min(t.g0 + wrow_last + wr, t.e - 1) : -1);
  const int wave_kmin = wave_uniform(t.g0 + w * 32 - wl);
  const int wave_gmin = wave_uniform(t.g0 + w * 32);
  const int wave_gmax = wave_uniform(t.g0 + w * 32 + 31);
  const bool wave_all_valid =
      wave_uniform((w * 32 + 31 < t.n) && (t.g0 + w * 32 + 31 < t.e)) != 0;

  // Staging by LDS DMA: DMA instruction j of wave w fills rows
  // [(w*NI + j)*RPI, +RPI) of a tile; lane i loads row (w*NI + j)*RPI +
  // i/LPR, physical chunk i%LPR, i.e. logical chunk (i%LPR) ^ dq_swz(row).
  // Rows at or past the end of the tile's key range read (and land as) 0
  // with no branch.
  //  - Unmapped: the descriptor runs from row k0 - kv_sub to the range end.
  //  - MAPPED: pos[] holds this lane's rows of a tile, looked up one tile
  //    ahead of the loads that use them, and a skipped row gets an offset
  //    past the descriptor, which spans all kv rows (below 2 GiB).
  const uint32_t row_bytes = (uint32_t)(rs * 2);
  int drow[NI];
  uint32_t dcol[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    drow[j] = (w * NI + j) * RPI + lane / LPR;
    dcol[j] = (uint32_t)(((lane % LPR) ^ dq_swz<D>(drow[j])) * 16);
  }
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
  auto load_tile = [&](int k0, int kend, const int (&pos)[NI], int buf) {
    if constexpr (MAPPED) {
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + head_off, kv_bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + head_off, kv_bytes);
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const uint32_t off = pos[j] >= 0 ? (uint32_t)pos[j] * row_bytes + dcol[j] : 0xFFFFFFF0u;
        dma16(rk, off, sm.k[buf] + (w * NI + j) * 1024);
        dma16(rv, off, sm.v[buf] + (w * NI + j) * 1024);
      }
    } else {
      const int64_t n = (int64_t)kend - k0;
      const uint32_t bytes = n > 0 ? (uint32_t)(n * rs * 2) : 0u;
      const int64_t base = n > 0 ? (int64_t)(k0 - kv_sub) * rs : 0;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + base + head_off, bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + base + head_off, bytes);
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const uint32_t off = (uint32_t)drow[j] * row_bytes + dcol[j];
        dma16(rk, off, sm.k[buf] + (w * NI + j) * 1024);
        dma16(rv, off, sm.v[buf] + (w * NI + j) * 1024);
      }
    }
  };
  // LDS byte offsets of this lane's K / V fragment reads (lane constants):
  // key block kb, k-step kk is row kb*32 + li, logical chunk 2kk + hh. (The
  // K^T reads' offsets are formed in the loop.)
  const int fsw = hh ^ dq_swz<D>(li);
  auto f_off = [&](int kb, int kk) {
    return (kb * 32 + li) * ROWB + (((2 * kk) ^ fsw) << 4);
  };

  // Key tiles: those of [ks0, ke0), then those of [ks1, ke1).
  const int nt0 = t.ke0 > t.ks0 ? (t.ke0 - t.ks0 + BN - 1) / BN : 0;
  const int nt1 = t.ke1 > t.ks1 ? (t.ke1 - t.ks1 + BN - 1) / BN : 0;
  const int ntiles = nt0 + nt1;
  auto tile_k0 = [&](int it) { return it < nt0 ? t.ks0 + it * BN : t.ks1 + (it - nt0) * BN; };
  auto tile_kend = [&](int it) { return it < nt0 ? t.ke0 : t.ke1; };
  // The second tile's rows are looked up beside the first's, so the prologue
  // waits on one row-map round trip before the first K/V loads, not two.
  int pos[NI], pos1[NI] = {};
  if (ntiles > 0) {
    rows_pos(tile_k0(0), tile_kend(0), pos);
    if (ntiles > 1) rows_pos(tile_k0(1), tile_kend(1), pos1);
    load_tile(tile_k0(0), tile_kend(0), pos, 0);
#pragma unroll
    for (int j = 0; j < NI; ++j) pos[j] = pos1[j];
  }
  wait_vmem();  // Q/dO fragments have landed: the loop's MFMAs never wait on loads
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int k0 = tile_k0(it);
    const int kend = tile_kend(it);
    const int cur = it & 1;
    const bool has_next = it + 1 < ntiles;
    if (has_next) {  // into the other buffer, whose last readers passed the previous barrier
      load_tile(tile_k0(it + 1), tile_kend(it + 1), pos, cur ^ 1);
      if (it + 2 < ntiles) rows_pos(tile_k0(it + 2), tile_kend(it + 2), pos);
    }

    if (k0 <= wave_kmax && (!BAND || k0 + BN - 1 >= wave_kmin)) {
      // With 8 waves over unmapped K/V, dP^T accumulates from -delta (this
      // lane's query), so the products leave dP^T - delta and dS^T =
      // P^T (dP^T - delta) is one multiply (dQ -3.5% on one 75600-token
      // document). Elsewhere the accumulators, live longer than zero-initialised
      // ones (whose first MFMA takes a literal 0), push the kernel into more
      // spilling (+18..39% with 4 waves on short-document shares), so they
      // start at 0 and delta is subtracted per element.
      constexpr bool kDeltaInit = WAVES == 8 && !MAPPED;
      f32x16 s[2], dp[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[kb][i] = 0.f;
          dp[kb][i] = kDeltaInit ? -dlt : 0.f;
        }
      // 16 steps (key block kb = n & 1, k-step kk = n >> 1), four independent
      // accumulator chains; each step's K and V fragments are read kPf steps
      // ahead into a ring, so an MFMA never waits on a read issued just
      // before it. The wave raises its priority over these products: on a
      // SIMD shared with another wave, their MFMAs issue ahead of that wave's
      // exponentials and dQ products (dQ -6.8% on one 75600-token document;
      // raised over the dQ product as well, -4.8%).
      constexpr int kPf = 2;
      constexpr int kSteps = 2 * KSTEPS;
      bf16x8 kr[kPf + 1], vr[kPf + 1];
      auto fetch = [&](int n) {
        const int off = f_off(n & 1, n >> 1);
        kr[n % (kPf + 1)] = load_bf16x8(reinterpret_cast<const bf16*>(&sm.k[cur][off]));
        vr[n % (kPf + 1)] = load_bf16x8(reinterpret_cast<const bf16*>(&sm.v[cur][off]));
      };
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int n = 0; n < kPf; ++n) fetch(n);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int n = 0; n < kSteps; ++n) {
        if (n + kPf < kSteps) fetch(n + kPf);
        const int kb = n & 1, kk = n >> 1;
        s[kb] = mfma32(kr[n % (kPf + 1)], qf[kk], s[kb]);
        dp[kb] = mfma32(vr[n % (kPf + 1)], dof[kk], dp[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      // Exponents S * scale_log2 - LSE_2. Tiles on a band edge or past the
      // range end (one wave-uniform test) give a masked key exponent -inf,
      // so p = 0 exactly with no branch (dP is finite: rows past the range
      // end load as zeros); the others skip the mask. A per-element
      // short-circuit test, or a select after the exp, compiled to a branch
      // around every element.
      const bool diag = wave_uniform(!wave_all_valid || k0 + BN - 1 > wave_gmin + wr ||
                                     (BAND && k0 < wave_gmax - wl) || k0 + BN > kend) != 0;
      if (diag) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + kb * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
            bool ok = (key <= my_hi) & (key < kend);
            if constexpr (BAND) ok &= key >= my_lo;
            s[kb][i] = ok ? fmaf(s[kb][i], scale_log2, -lse2) : -INFINITY;
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[kb][i] = fmaf(s[kb][i], scale_log2, -lse2);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(s[kb][i]);
          dp[kb][i] = p * (kDeltaInit ? dp[kb][i] : dp[kb][i] - dlt);
        }
      // dQ^T += K^T dS^T; k-step (kb, u): slot j = key kb*32 + 16u +
      // (j/4)*8 + hh*4 + j%4 (accumulator entries u*8..u*8+7 of dp[kb]).
      // 4 * DB MFMAs (m = (kb, u, db)), their K^T operands read kPf ahead.
      bf16x8 dsb[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u) dsb[kb * 2 + u] = to_bf16x8(dp[kb], u * 8);
      constexpr int kMs = 4 * DB;
      // The transposing reads' lane offsets, recomputed per tile from a copy
      // of the lane index the compiler cannot see through (an empty asm
      // statement), so they are not held in registers across the whole loop:
      // hoisted, they were spilled and reloaded inside it, and the reloads'
      // waits also waited for the next tile's loads (dQ -0.5..1% on one
      // 75600-token document; recomputing the K/V fragment offsets as well
      // removed every spill but cost 8%, the address arithmetic landing among
      // the S/dP MFMAs).
      int lane_o = lane;
      asm volatile("" : "+v"(lane_o));
      const int sl_o = lane_o & 15, g16_o = (lane_o >> 4) & 3, hh_o = (lane_o >> 5) & 1;
      const int tr_o = hh_o * 4 + (sl_o >> 2);
      const int tb_o = 2 * (g16_o & 1) + ((sl_o & 3) >> 1);
      const int tsw0_o = tb_o ^ dq_swz<D>(tr_o), tsw1_o = tb_o ^ dq_swz<D>(tr_o + 8);
      const int tbase_o = tr_o * ROWB + 8 * (sl_o & 1);
      // K^T read of key block kb, half u, head-dim block db: rows kb*32 + 16u
      // + 4hh + (sl >> 2) (+8), logical chunk 4db + 2(g16 & 1) + ((sl & 3) >>
      // 1), half sl & 1.
      auto t_off_o = [&](int kb, int u, int half, int db) {
        return tbase_o + (kb * 32 + 16 * u + 8 * half) * ROWB +
               (((4 * db) ^ (half ? tsw1_o : tsw0_o)) << 4);
      };
      bf16x8 ar[kPf + 1];
      auto fetch_t = [&](int m) {
        const int kb = m / (2 * DB), u = (m / DB) & 1, db = m % DB;
        ar[m % (kPf + 1)] =
            concat4(lds_read_tr4(reinterpret_cast<const bf16*>(&sm.k[cur][t_off_o(kb, u, 0, db)])),
                    lds_read_tr4(reinterpret_cast<const bf16*>(&sm.k[cur][t_off_o(kb, u, 1, db)])));
      };
#pragma unroll
      for (int m = 0; m < kPf; ++m) fetch_t(m);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < kMs; ++m) {
        if (m + kPf < kMs) fetch_t(m + kPf);
        acc[m % DB] = mfma32(ar[m % (kPf + 1)], dsb[m / DB], acc[m % DB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    wait_vmem();  // this wave's DMA of the next tile has landed
    __syncthreads();
  }

  if (t.nparts > 1) {
    // Split key walk: this part's accumulators go to its scratch slot in lane
    // order; the last part to finish sums all parts in part order.
    auto acc_at = [&](int x, int db, int i4) {
      return reinterpret_cast<f32x4*>(split_slot<D, WAVES * 32>(split.part, x, h, H)) +
             ((db * 4 + i4) * kThreads + threadIdx.x);
    };
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 a;
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = acc[db][i4 * 4 + j];
        *acc_at(t.slot + t.part, db, i4) = a;
      }
    if (!split_arrive(split.cnt + (int64_t)t.group * H + h, t.nparts)) return;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 a = *acc_at(t.slot, db, i4);
        for (int p = 1; p < t.nparts; ++p) {
          const f32x4 b = *acc_at(t.slot + p, db, i4);
#pragma unroll
          for (int j = 0; j < 4; ++j) a[j] += b[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[db][i4 * 4 + j] = a[j];
      }
  }

  if (!in_tile) return;
  float* qp = dq + m * rs + head_off;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      f32x4 out;
#pragma unroll
      for (int j = 0; j < 4; ++j) out[j] = acc[db][i4 * 4 + j] * scale;
      f32x4* dst = reinterpret_cast<f32x4*>(qp + db * 32 + i4 * 8 + hh * 4);
      if (accumulate) {
        const f32x4 cur = *dst;
#pragma unroll
        for (int j = 0; j < 4; ++j) out[j] += cur[j];
      }
      *dst = out;
    }
}

}  // namespace

namespace {

template <int D, int WAVES, bool M>
void launch_dq_dm(int64_t blocks, hipStream_t stream, const FwdTile* tiles, int32_t H,
                  const bf16* q, const bf16* k, const bf16* v, const int32_t* kv_row,
                  int32_t kv_sub, uint32_t kvb, Band band, const bf16* d_o, const bf16* o,
                  const float* lse, float* delta, float* dq, int64_t n_local, float scale,
                  int32_t accumulate, int32_t n_attn, SplitWs split, const DqExtras& ex) {
#define THDCP_DQ(DL, BB)                                                                      \
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, WAVES, M, DL, BB>), dim3((unsigned)blocks),          \
                     dim3(WAVES * 64),                                                         \
                     0, stream, tiles, H, q, k, v, kv_row, kv_sub, kvb, band.wl, band.wr, d_o,  \
                     o, lse, delta, dq, n_local, accumulate, scale, scale * kLog2e, n_attn, split,  \
                     ex)
  if (o && band.causal)
    THDCP_DQ(true, false);
  else if (o)
    THDCP_DQ(true, true);
  else if (band.causal)
    THDCP_DQ(false, false);
  else
    THDCP_DQ(false, true);
#undef THDCP_DQ
}

}  // namespace

hipError_t launch_attn_bwd_dq(const FwdTile* tiles, int32_t n_tiles, int32_t H, int32_t D,
                              int32_t rows, const void* q, const void* k, const void* v, KvRows kv,
                              Band band, const void* d_o, const void* o, const float* lse,
                              float* delta, float* dq, int64_t n_local, float scale,
                              int32_t accumulate, SplitWs split, const DqExtras& ex,
                              hipStream_t stream) {
  const int64_t attn_blocks = (int64_t)n_tiles * H;
  const int64_t zero_blocks =
      (ex.zr && ex.n_zr > 0) ? (ex.zero_rows + kZeroRowsPerBlock - 1) / kZeroRowsPerBlock : 0;
  const int64_t blocks = attn_blocks + zero_blocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const bf16* qb = static_cast<const bf16*>(q);
  const bf16* kb = static_cast<const bf16*>(k);
  const bf16* vb = static_cast<const bf16*>(v);
  const bf16* db = static_cast<const bf16*>(d_o);
  const bf16* ob = static_cast<const bf16*>(o);
  const int64_t kv_bytes = kv.rows * H * D * 2;
  if (kv.map && kv_bytes >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const uint32_t kvb = kv.map ? (uint32_t)kv_bytes : 0u;
  const int32_t sub = (int32_t)kv.sub;
#define THDCP_DQ_D(DD, WW, MM)                                                                 \
  launch_dq_dm<DD, WW, MM>(blocks, stream, tiles, H, qb, kb, vb, kv.map, sub, kvb, band, db, ob,  \
                           lse, delta, dq, n_local, scale, accumulate, (int32_t)attn_blocks,     \
                           split, ex)
  const bool mm = kv.map != nullptr;
  if (D == 128 && rows == kFwdBM)
    mm ? THDCP_DQ_D(128, 4, true) : THDCP_DQ_D(128, 4, false);
  else if (D == 128 && rows == kFwdBMLong)
    mm ? THDCP_DQ_D(128, 8, true) : THDCP_DQ_D(128, 8, false);
  else if (D == 64 && rows == kFwdBM)
    mm ? THDCP_DQ_D(64, 4, true) : THDCP_DQ_D(64, 4, false);
  else if (D == 64 && rows == kFwdBMLong)
    mm ? THDCP_DQ_D(64, 8, true) : THDCP_DQ_D(64, 8, false);
#undef THDCP_DQ_D
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace thdcp
