// lora_fwd.hip -- shrink / expand / fused multi-adapter LoRA kernels for gfx950.
//
// Method: every token of a batch carries an adapter; the batch is cut into
// segments of one adapter each and a single launch covers all of them (C-LoRA
// announcement, "Come funziona l'architettura"). Work is tiled along the
// token (sequence) and hidden dimensions, never along the small rank (PLoRA
// summary, "Kernelontwerp"). The same kernel serves the backward du/dx pass
// with dy in place of x, B^T in place of A and A^T in place of B.
//
// Shapes handled by one workgroup (4 wave64):
//  shrink  P^T[rank 32b..32b+31][token 0..31] += W[rank][k] * X[token][k]
//          32x32x16 bf16 MFMA; both operands are read straight from global
//          memory with 16-byte loads (8 consecutive k per lane); the 4 waves
//          split k and are summed in LDS in a fixed order.
//  expand  Y^T[col][token] += V[col][rank] * P^T[rank][token]
//          32x32x16 bf16 MFMA; P (fp32) enters as a bf16 hi + lo pair; rows
//          of each 32-column block are permuted (colmap) so that every lane
//          owns two runs of 8 contiguous bf16 of one token row of Y.
#include "lora_device.h"
#include "lora_plan.h"

namespace lora {

constexpr int kLdp = 128 + 4;  // LDS row length of the P tile (floats)

struct TileInfo {
  int g;       // global tile index in the plan
  int p0;      // first sorted position of the tile
  int cnt;     // valid tokens in the tile (1..32)
  int adapter;
  int rank;
  int slot;
  float scale;
};

__device__ __forceinline__ TileInfo tile_info(const FwdPlan& P, int g) {
  int lo = 0, hi = P.n_seg;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (P.seg_tile0[mid] <= g) lo = mid; else hi = mid;
  }
  TileInfo t;
  t.g = g;
  const int tt = g - P.seg_tile0[lo];
  t.p0 = P.seg_tok0[lo] + tt * kTileM;
  t.cnt = min(kTileM, P.seg_ntok[lo] - tt * kTileM);
  t.adapter = P.seg_adapter[lo];
  t.rank = P.seg_rank[lo];
  t.slot = P.seg_slot[lo];
  t.scale = P.seg_scale[lo];
  return t;
}

__device__ __forceinline__ const uint16_t* w_ptr(const FwdPlan& P, const TileInfo& t) {
  if (P.Wtab) return reinterpret_cast<const uint16_t*>(P.Wtab[t.adapter]);
  return P.Wslots + (int64_t)t.slot * P.w_slot_elems;
}
__device__ __forceinline__ const uint16_t* v_ptr(const FwdPlan& P, const TileInfo& t) {
  if (P.Vtab) return reinterpret_cast<const uint16_t*>(P.Vtab[t.adapter]);
  return P.Vslots + (int64_t)t.slot * P.v_slot_elems;
}

// Row of X / Y used by sorted position p.
__device__ __forceinline__ int64_t token_row(const FwdPlan& P, int p) {
  return P.token_rows ? (int64_t)P.token_rows[p] : (int64_t)p;
}

// ---------------------------------------------------------------------------
// Shrink: acc[b] (rows = rank 32b.., cols = this lane's token) over k in [kb, ke)
// ---------------------------------------------------------------------------
template <int RB, int UNR>
__device__ __forceinline__ void shrink_acc(const uint16_t* xrow, bool xvalid, const uint16_t* W,
                                           int64_t ldw, int rank, int kb, int ke, int wave,
                                           int lane, f32x16 (&acc)[RB]) {
  const int h = lane >> 5, m = lane & 31;
  const uint16_t* wrow[RB];
  bool wv[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int row = 32 * b + m;
    wv[b] = row < rank;
    wrow[b] = W + (int64_t)(wv[b] ? row : 0) * ldw;
  }
  constexpr int kUnit = 16 * UNR;
  for (int k0 = kb + wave * kUnit; k0 < ke; k0 += 4 * kUnit) {
    u32x4 xf[UNR], wf[RB][UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int k = k0 + 16 * u + 8 * h;
      const bool kv = k < ke;
      xf[u] = (xvalid && kv) ? ld16(xrow + k) : zero16();
#pragma unroll
      for (int b = 0; b < RB; ++b) wf[b][u] = (wv[b] && kv) ? ld16(wrow[b] + k) : zero16();
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u)
#pragma unroll
      for (int b = 0; b < RB; ++b) acc[b] = mfma32(as_bf16x8(wf[b][u]), as_bf16x8(xf[u]), acc[b]);
  }
}

// Sum acc over the 4 waves (fixed order 0,1,2,3) and hand every element
// (rank row k, token n, value) to `out`. red: LDS float[4 * 16 * 64].
template <int RB, typename F>
__device__ __forceinline__ void reduce_waves(float* red, const f32x16 (&acc)[RB], int wave,
                                             int lane, F&& out) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[(wave * 16 + i) * 64 + lane] = acc[b][i];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid + 256 * j;
      const int ln = e & 63, i = e >> 6;
      float s = red[(0 * 16 + i) * 64 + ln];
      s += red[(1 * 16 + i) * 64 + ln];
      s += red[(2 * 16 + i) * 64 + ln];
      s += red[(3 * 16 + i) * 64 + ln];
      const int mm = 8 * (i >> 2) + 4 * (ln >> 5) + (i & 3);
      out(32 * b + mm, ln & 31, s);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Expand
// ---------------------------------------------------------------------------
template <int RB>
struct PFrags {
  bf16x8 hi[2 * RB];
  bf16x8 lo[2 * RB];
};

// B-operand fragments of P^T from the LDS tile Pl[token][k]: lane supplies
// P[token = lane%32][16kb + 8(lane/32) + e].
template <int RB>
__device__ __forceinline__ void build_pfrags(const float* Pl, int rank, int lane, PFrags<RB>& F) {
  const int n = lane & 31, h = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 2 * RB; ++kb) {
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = 16 * kb + 8 * h + e;
      f[e] = (k < rank) ? Pl[n * kLdp + k] : 0.f;
    }
    split8(f, F.hi[kb], F.lo[kb]);
  }
}

// 8 bf16 of row `row` starting at k, zero beyond `rank`, for rows whose
// stride is not a multiple of 8 elements.
__device__ __forceinline__ u32x4 ld_partial(const uint16_t* row, int k, int rank) {
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t a = (k + 2 * q < rank) ? row[k + 2 * q] : 0u;
    const uint32_t b = (k + 2 * q + 1 < rank) ? row[k + 2 * q + 1] : 0u;
    w[q] = a | (b << 16);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// y[token][col] += oscale * sum_k V[col][k] P[token][k] for column blocks
// [cb_begin, cb_end) handled round-robin by the 4 waves.
template <int RB>
__device__ __forceinline__ void expand_run(const PFrags<RB>& F, const uint16_t* V, int64_t ldv,
                                           int rank, bool vec16, int ncols, uint16_t* yrow,
                                           bool yvalid, int cb_begin, int cb_end, float oscale,
                                           int wave, int lane) {
  const int m = lane & 31, h = lane >> 5;
  const int kbn = (rank + 15) >> 4;
  for (int cb = cb_begin + wave; cb < cb_end; cb += 4) {
    const int col0 = cb * 32;
    const int vcol = col0 + colmap(m);
    const bool vok = vcol < ncols;
    const uint16_t* vrow = V + (int64_t)(vok ? vcol : 0) * ldv;
    u32x4 vf[2 * RB];
#pragma unroll
    for (int kb = 0; kb < 2 * RB; ++kb) {
      const int k = 16 * kb + 8 * h;
      if (kb < kbn && vok && k < rank)
        vf[kb] = vec16 ? ld16(vrow + k) : ld_partial(vrow, k, rank);
      else
        vf[kb] = zero16();
    }
    const int c0 = col0 + 8 * h, c1 = col0 + 16 + 8 * h;
    const bool ok0 = yvalid && c0 < ncols, ok1 = yvalid && c1 < ncols;
    const u32x4 y0 = ok0 ? ld16(yrow + c0) : zero16();
    const u32x4 y1 = ok1 ? ld16(yrow + c1) : zero16();
    f32x16 acc = zero_acc16();
#pragma unroll
    for (int kb = 0; kb < 2 * RB; ++kb) {
      if (kb < kbn) {
        acc = mfma32(as_bf16x8(vf[kb]), F.hi[kb], acc);
        acc = mfma32(as_bf16x8(vf[kb]), F.lo[kb], acc);
      }
    }
    float f[8];
    if (ok0) {
      unpack8(y0, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = f[i] + oscale * acc[i];
      st16(yrow + c0, pack8(f));
    }
    if (ok1) {
      unpack8(y1, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = f[i] + oscale * acc[8 + i];
      st16(yrow + c1, pack8(f));
    }
  }
}

// ---------------------------------------------------------------------------
// Items
// ---------------------------------------------------------------------------
struct Smem {
  float red[4 * 16 * 64];
  float Pl[kTileM * kLdp];
  int flag;
};

template <int RB>
__device__ __forceinline__ int unroll_for() {
  return RB == 1 ? 8 : (RB == 2 ? 4 : 2);
}

template <int RB>
__device__ __forceinline__ void shrink_range(const FwdPlan& P, const TileInfo& t, int kb, int ke,
                                             int wave, int lane, f32x16 (&acc)[RB]) {
  const int n = lane & 31;
  const bool xvalid = n < t.cnt;
  const uint16_t* xrow = P.X + (xvalid ? token_row(P, t.p0 + n) : 0) * P.ldx;
#pragma unroll
  for (int b = 0; b < RB; ++b) acc[b] = zero_acc16();
  constexpr int UNR = RB == 1 ? 8 : (RB == 2 ? 4 : 2);
  shrink_acc<RB, UNR>(xrow, xvalid, w_ptr(P, t), P.K, t.rank, kb, ke, wave, lane, acc);
}

// Writes Pl rows 0..31, columns < 32*RB (zero where rank/token invalid) to U.
__device__ __forceinline__ void store_u_from_lds(const FwdPlan& P, const TileInfo& t,
                                                 const float* Pl) {
  for (int e = threadIdx.x; e < kTileM * t.rank; e += kThreads) {
    const int n = e / t.rank, k = e - n * t.rank;
    if (n < t.cnt) P.U[(int64_t)(t.p0 + n) * P.ldu + k] = Pl[n * kLdp + k];
  }
}

template <int RB>
__device__ __forceinline__ void expand_tile_from_lds(const FwdPlan& P, const TileInfo& t, int c,
                                                     const float* Pl, int wave, int lane) {
  PFrags<RB> F;
  build_pfrags<RB>(Pl, t.rank, lane, F);
  const int n = lane & 31;
  const bool yvalid = n < t.cnt;
  uint16_t* yrow = P.Y + (yvalid ? token_row(P, t.p0 + n) : 0) * P.ldy;
  const int nblocks = (P.N + 31) >> 5;
  const int cb0 = c * P.nblk;
  const int cb1 = min(nblocks, cb0 + P.nblk);
  const int ldv = ((t.rank + P.v_round - 1) / P.v_round) * P.v_round;
  const bool vec16 = (ldv & 7) == 0;
  const float oscale = P.scale_in_shrink ? 1.f : t.scale;
  expand_run<RB>(F, v_ptr(P, t), ldv, t.rank, vec16, P.N, yrow, yvalid, cb0, cb1, oscale, wave,
                 lane);
}

// kModeFusedTile: full shrink of one tile on chip, then its n-chunk c.
template <int RB>
__device__ __forceinline__ void item_fused_tile(const FwdPlan& P, Smem& S, const TileInfo& t, int c) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  f32x16 acc[RB];
  shrink_range<RB>(P, t, 0, P.K, wave, lane, acc);
  const float ps = P.scale_in_shrink ? t.scale : 1.f;
  float* Pl = S.Pl;
  reduce_waves<RB>(S.red, acc, wave, lane, [&](int k, int n, float v) { Pl[n * kLdp + k] = v * ps; });
  if (P.write_u && c == 0) store_u_from_lds(P, t, Pl);
  expand_tile_from_lds<RB>(P, t, c, Pl, wave, lane);
}

// kModeExpand: U from memory, expand n-chunk c.
template <int RB>
__device__ __forceinline__ void item_expand(const FwdPlan& P, Smem& S, const TileInfo& t, int c) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* Pl = S.Pl;
  for (int e = threadIdx.x; e < kTileM * 32 * RB; e += kThreads) {
    const int n = e / (32 * RB), k = e - n * (32 * RB);
    Pl[n * kLdp + k] = (n < t.cnt && k < t.rank) ? P.U[(int64_t)(t.p0 + n) * P.ldu + k] : 0.f;
  }
  __syncthreads();
  expand_tile_from_lds<RB>(P, t, c, Pl, wave, lane);
}

__device__ __forceinline__ float* partial_ptr(const FwdPlan& P, int g, int c) {
  return P.partials + ((int64_t)g * P.ks + c) * kTileM * P.rpad;
}

// kModeShrink / kModeFusedDep phase A: shrink over k-chunk c.
template <int RB>
__device__ __forceinline__ void item_shrink(const FwdPlan& P, Smem& S, const TileInfo& t, int c) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kb = c * P.kchunk;
  const int ke = min(P.K, kb + P.kchunk);
  f32x16 acc[RB];
  shrink_range<RB>(P, t, kb, ke, wave, lane, acc);
  const float ps = P.scale_in_shrink ? t.scale : 1.f;
  if (P.mode == kModeShrink && P.ks == 1) {
    reduce_waves<RB>(S.red, acc, wave, lane, [&](int k, int n, float v) {
      if (n < t.cnt && k < t.rank) P.U[(int64_t)(t.p0 + n) * P.ldu + k] = v * ps;
    });
    return;
  }
  float* part = partial_ptr(P, t.g, c);
  const int rpad = P.rpad;
  reduce_waves<RB>(S.red, acc, wave, lane, [&](int k, int n, float v) { part[n * rpad + k] = v; });
  // publish the partial: every thread's stores, then one counter increment
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  int* ctr = P.counters + kCtrTiles + t.g;
  if (P.mode == kModeFusedDep) {
    if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  // kModeShrink, ks > 1: the last arriving chunk sums all chunks in order
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    S.flag = (old == P.ks - 1);
  }
  __syncthreads();
  if (!S.flag) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  for (int e = threadIdx.x; e < kTileM * t.rank; e += kThreads) {
    const int n = e / t.rank, k = e - n * t.rank;
    if (n >= t.cnt) continue;
    float s = partial_ptr(P, t.g, 0)[n * rpad + k];
    for (int q = 1; q < P.ks; ++q) s += partial_ptr(P, t.g, q)[n * rpad + k];
    P.U[(int64_t)(t.p0 + n) * P.ldu + k] = s * ps;
  }
  if (threadIdx.x == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// kModeFusedDep phase B: wait for the tile's k-chunks, sum them, expand.
// If the chunks do not arrive within spin_ticks (e.g. their workgroups are
// not resident), the item computes the same chunks itself in the same order,
// so the result is identical and no wait is unbounded.
template <int RB>
__device__ __forceinline__ void item_expand_wait(const FwdPlan& P, Smem& S, const TileInfo& t, int c) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int* ctr = P.counters + kCtrTiles + t.g;
  if (threadIdx.x == 0) {
    const uint64_t t0 = wall_clock64();
    int ready = 0;
    while (true) {
      if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= P.ks) { ready = 1; break; }
      if (wall_clock64() - t0 > (uint64_t)P.spin_ticks) break;
      __builtin_amdgcn_s_sleep(1);
    }
    S.flag = ready;
  }
  __syncthreads();
  const float ps = P.scale_in_shrink ? t.scale : 1.f;
  float* Pl = S.Pl;
  const int rcols = 32 * RB;
  if (S.flag) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const int rpad = P.rpad;
    for (int e = threadIdx.x; e < kTileM * rcols; e += kThreads) {
      const int n = e / rcols, k = e - n * rcols;
      float s = partial_ptr(P, t.g, 0)[n * rpad + k];
      for (int q = 1; q < P.ks; ++q) s += partial_ptr(P, t.g, q)[n * rpad + k];
      Pl[n * kLdp + k] = s * ps;
    }
  } else {
    for (int q = 0; q < P.ks; ++q) {
      const int kb = q * P.kchunk;
      const int ke = min(P.K, kb + P.kchunk);
      f32x16 acc[RB];
      shrink_range<RB>(P, t, kb, ke, wave, lane, acc);
      reduce_waves<RB>(S.red, acc, wave, lane, [&](int k, int n, float v) {
        Pl[n * kLdp + k] = (q == 0) ? v : Pl[n * kLdp + k] + v;
      });
    }
    for (int e = threadIdx.x; e < kTileM * rcols; e += kThreads) {
      const int n = e / rcols, k = e - n * rcols;
      Pl[n * kLdp + k] *= ps;
    }
  }
  __syncthreads();
  if (P.write_u && c == 0) store_u_from_lds(P, t, Pl);
  expand_tile_from_lds<RB>(P, t, c, Pl, wave, lane);
}

template <int RB>
__device__ __forceinline__ void run_item(const FwdPlan& P, Smem& S, const TileInfo& t, int kind, int c) {
  switch (kind) {
    case 0: item_shrink<RB>(P, S, t, c); break;
    case 1: item_expand<RB>(P, S, t, c); break;
    case 2: item_fused_tile<RB>(P, S, t, c); break;
    default: item_expand_wait<RB>(P, S, t, c); break;
  }
}

__global__ __launch_bounds__(kThreads) void sgmv_fwd_kernel(FwdPlan P) {
  __shared__ Smem S;
  const int b = blockIdx.x;
  int item = -1, kind = 0, per = 1;
  if (P.mode == kModeFusedDep) {
    if (b < P.n_items_a) { item = b; kind = 0; per = P.ks; }
    else if (b < P.n_items_a + P.n_items_b) { item = b - P.n_items_a; kind = 3; per = P.nc; }
  } else {
    int it = b;
    if (P.xcd_remap) {
      const int q = P.grid >> 3;
      it = (b & 7) * q + (b >> 3);
    }
    if (it < P.n_items_a) item = it;
    kind = P.mode == kModeShrink ? 0 : (P.mode == kModeExpand ? 1 : 2);
    per = P.mode == kModeShrink ? P.ks : P.nc;
  }
  if (item >= 0) {
    const int g = item / per, c = item - g * per;
    const TileInfo t = tile_info(P, g);
    if (t.rank <= 32) run_item<1>(P, S, t, kind, c);
    else if (t.rank <= 64) run_item<2>(P, S, t, kind, c);
    else run_item<4>(P, S, t, kind, c);
  }
  if (P.mode == kModeFusedDep) {
    // the last workgroup to finish returns every counter of this launch to zero
    __syncthreads();
    if (threadIdx.x == 0) {
      const int old = __hip_atomic_fetch_add(P.counters + kCtrDone, 1, __ATOMIC_ACQ_REL,
                                             __HIP_MEMORY_SCOPE_AGENT);
      if (old == P.grid - 1) {
        for (int g = 0; g < P.n_tiles; ++g)
          __hip_atomic_store(P.counters + kCtrTiles + g, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(P.counters + kCtrDone, 0, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

hipError_t launch_fwd(const FwdPlan& P, hipStream_t stream) {
  hipLaunchKernelGGL(sgmv_fwd_kernel, dim3(P.grid), dim3(kThreads), 0, stream, P);
  return hipGetLastError();
}

}  // namespace lora
