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

// Finds the segment that holds tile g with one parallel read of the segment
// table: thread i checks segment i and the matching thread publishes the
// tile's description in LDS (a binary search would chain several dependent
// loads of the kernel-argument table).
template <typename PT>
__device__ __forceinline__ TileInfo tile_info(const PT& P, int g, TileInfo* lds) {
  const int i = threadIdx.x;
  if (i < P.n_seg) {
    const int t0 = P.seg_tile0[i];
    const int t1 = (i + 1 < P.n_seg) ? P.seg_tile0[i + 1] : P.n_tiles;
    const int tok0 = P.seg_tok0[i], ntok = P.seg_ntok[i];
    const int adapter = P.seg_adapter[i], rank = P.seg_rank[i], slot = P.seg_slot[i];
    const float scale = P.seg_scale[i];
    if (g >= t0 && g < t1) {
      const int tt = g - t0;
      TileInfo t;
      t.g = g;
      t.p0 = tok0 + tt * kTileM;
      t.cnt = min(kTileM, ntok - tt * kTileM);
      t.adapter = adapter;
      t.rank = rank;
      t.slot = slot;
      t.scale = scale;
      *lds = t;
    }
  }
  __syncthreads();
  TileInfo t = *lds;
  t.g = __builtin_amdgcn_readfirstlane(t.g);
  t.p0 = __builtin_amdgcn_readfirstlane(t.p0);
  t.cnt = __builtin_amdgcn_readfirstlane(t.cnt);
  t.adapter = __builtin_amdgcn_readfirstlane(t.adapter);
  t.rank = __builtin_amdgcn_readfirstlane(t.rank);
  t.slot = __builtin_amdgcn_readfirstlane(t.slot);
  t.scale = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, t.scale)));
  return t;
}

template <typename PT>
__device__ __forceinline__ const uint16_t* w_ptr(const PT& P, const TileInfo& t) {
  if (P.Wtab) return reinterpret_cast<const uint16_t*>(P.Wtab[t.adapter]);
  return P.Wslots + (int64_t)t.slot * P.w_slot_elems;
}
template <typename PT>
__device__ __forceinline__ const uint16_t* v_ptr(const PT& P, const TileInfo& t) {
  if (P.Vtab) return reinterpret_cast<const uint16_t*>(P.Vtab[t.adapter]);
  return P.Vslots + (int64_t)t.slot * P.v_slot_elems;
}

// Row of X / Y used by sorted position p.
template <typename PT>
__device__ __forceinline__ int64_t token_row(const PT& P, int p) {
  return P.token_rows ? (int64_t)P.token_rows[p] : (int64_t)p;
}

// ---------------------------------------------------------------------------
// Shrink: acc[b] (rows = rank 32b.., cols = this lane's token) over k in [kb, ke)
// ---------------------------------------------------------------------------
// Ring depth of the shrink loop (k-steps of 16 whose loads are in flight).
template <int RB>
struct ShrinkDepth {
  static constexpr int v = RB == 1 ? 8 : (RB == 2 ? 6 : 4);
};
// xr: resource over the tile's X rows; xoff: byte offset of this lane's token
// row (kOff if the token is not valid). W rows of rank >= rank fall outside
// the W resource and read as zero.
template <int RB>
__device__ __forceinline__ void shrink_acc(__amdgpu_buffer_rsrc_t xr, uint32_t xoff, const uint16_t* W,
                                           int64_t ldw, int rank, int kb, int ke, int wave,
                                           int lane, f32x16 (&acc)[RB]) {
  constexpr int DS = ShrinkDepth<RB>::v;
  const int h = lane >> 5, m = lane & 31;
  const __amdgpu_buffer_rsrc_t wr = mk_rsrc(W, (int64_t)rank * ldw * 2);
  uint32_t woff[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) woff[b] = (uint32_t)((int64_t)(32 * b + m) * ldw * 2);
  // each wave takes a contiguous quarter of [kb, ke) (multiple of 16 long)
  const int q = ((ke - kb + 63) >> 6) << 4;
  const int kw0 = __builtin_amdgcn_readfirstlane(kb + wave * q);
  const int kw1 = __builtin_amdgcn_readfirstlane(min(ke, kw0 + q));
  const int nsteps = __builtin_amdgcn_readfirstlane(kw1 > kw0 ? (kw1 - kw0 + 15) >> 4 : 0);
  u32x4 xf[DS], wf[RB][DS];
  auto load = [&](int j, int s) {
    const int k = kw0 + 16 * j + 8 * h;
    const bool kv = j < nsteps && k < kw1;
    xf[s] = bld16(xr, kv ? xoff + 2u * (uint32_t)k : kOff);
#pragma unroll
    for (int b = 0; b < RB; ++b) wf[b][s] = bld16(wr, kv ? woff[b] + 2u * (uint32_t)k : kOff);
  };
  // ring: DS k-steps of loads stay in flight while earlier ones are consumed
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    load(s, s);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int j0 = 0; j0 < nsteps; j0 += DS) {
#pragma unroll
    for (int s = 0; s < DS; ++s) {
#pragma unroll
      for (int b = 0; b < RB; ++b) acc[b] = mfma32(as_bf16x8(wf[b][s]), as_bf16x8(xf[s]), acc[b]);
      load(j0 + s + DS, s);
      // keep slot order: the refill of slot s is issued before slot s+1 is
      // consumed, so only slot s+1's own loads need to have arrived
      __builtin_amdgcn_sched_barrier(0);
    }
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

// One 32-column block of the expand as held in registers by a lane: the
// A-operand rows of V and the two 16-byte runs of this lane's y row.
template <int RB>
struct ExpBlock {
  u32x4 vf[2 * RB];
  u32x4 y0, y1;
  int cb;  // block index, -1 if none
};

struct ExpArgs {
  __amdgpu_buffer_rsrc_t vr;  // V [ncols, ldv] bf16
  int64_t ldv;
  int rank;
  bool vec16;
  int ncols;
  __amdgpu_buffer_rsrc_t yr;  // y rows of the tile
  uint32_t yoff;              // this lane's y row (kOff if invalid)
  float oscale;
};

template <int RB>
__device__ __forceinline__ void exp_load(const ExpArgs& a, int cb, int lane, ExpBlock<RB>& B) {
  const int m = lane & 31, h = lane >> 5;
  B.cb = cb;
  const int col0 = cb * 32;
  const uint32_t vrow = (uint32_t)((int64_t)(col0 + colmap(m)) * a.ldv * 2);  // rows >= ncols: outside
  const int kbn = (a.rank + 15) >> 4;  // k-steps of 16 that hold rank columns (uniform)
#pragma unroll
  for (int kb = 0; kb < 2 * RB; ++kb) {
    const int k = 16 * kb + 8 * h;
    if (kb >= kbn) {
      B.vf[kb] = zero16();  // never used by the MFMAs: no load issued
    } else if (a.vec16) {
      B.vf[kb] = bld16(a.vr, k < a.rank ? vrow + 2u * k : kOff);
    } else {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k0 = k + 2 * q;
        const uint32_t lo = bld2(a.vr, k0 < a.rank ? vrow + 2u * k0 : kOff);
        const uint32_t hi = bld2(a.vr, k0 + 1 < a.rank ? vrow + 2u * (k0 + 1) : kOff);
        w[q] = (lo & 0xffffu) | (hi << 16);
      }
      B.vf[kb] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
  const int c0 = col0 + 8 * h, c1 = col0 + 16 + 8 * h;
  B.y0 = bld16(a.yr, c0 < a.ncols ? a.yoff + 2u * c0 : kOff);
  B.y1 = bld16(a.yr, c1 < a.ncols ? a.yoff + 2u * c1 : kOff);
}

template <int RB>
__device__ __forceinline__ void exp_finish(const ExpArgs& a, const PFrags<RB>& F, int lane,
                                           const ExpBlock<RB>& B) {
  const int h = lane >> 5;
  const int kbn = (a.rank + 15) >> 4;
  f32x16 acc = zero_acc16();
#pragma unroll
  for (int kb = 0; kb < 2 * RB; ++kb) {
    if (kb < kbn) {
      acc = mfma32(as_bf16x8(B.vf[kb]), F.hi[kb], acc);
      acc = mfma32(as_bf16x8(B.vf[kb]), F.lo[kb], acc);
    }
  }
  const int col0 = B.cb * 32;
  const int c0 = col0 + 8 * h, c1 = col0 + 16 + 8 * h;
  float f[8];
  unpack8(B.y0, f);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = f[i] + a.oscale * acc[i];
  bst16(a.yr, c0 < a.ncols ? a.yoff + 2u * c0 : kOff, pack8(f));
  unpack8(B.y1, f);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = f[i] + a.oscale * acc[8 + i];
  bst16(a.yr, c1 < a.ncols ? a.yoff + 2u * c1 : kOff, pack8(f));
}

// Blocks per round of the expand loop (32-column blocks whose loads a wave
// issues together). Stores share the memory counter with loads on this chip
// family, so a pending y store would force every later wait to drain all
// loads; the expand therefore runs in rounds: issue a round's loads, wait
// once, then compute and store the round.
template <int RB>
struct ExpandDepth {
  static constexpr int v = RB == 1 ? 8 : (RB == 2 ? 4 : 2);
};

template <int RB>
struct ExpRing {
  ExpBlock<RB> b[ExpandDepth<RB>::v];
};

// Loads the round of blocks cb_first, cb_first + 4, ... (< cb_end).
template <int RB>
__device__ __forceinline__ void exp_ring_load(const ExpArgs& a, int cb_first, int cb_end, int lane,
                                              ExpRing<RB>& R) {
  constexpr int DE = ExpandDepth<RB>::v;
#pragma unroll
  for (int s = 0; s < DE; ++s) {
    const int cb = cb_first + 4 * s;
    if (cb < cb_end) {
      exp_load<RB>(a, cb, lane, R.b[s]);
    } else {
      R.b[s].cb = -1;
#pragma unroll
      for (int kb = 0; kb < 2 * RB; ++kb) R.b[s].vf[kb] = zero16();
      R.b[s].y0 = zero16();
      R.b[s].y1 = zero16();
    }
  }
}

// y[token][col] += oscale * sum_k V[col][k] P[token][k] over the wave's
// blocks; R holds the first round (already issued by the caller).
template <int RB>
__device__ __forceinline__ void exp_ring_run(const ExpArgs& a, const PFrags<RB>& F, int cb_first,
                                             int cb_end, int lane, ExpRing<RB>& R) {
  constexpr int DE = ExpandDepth<RB>::v;
  int cb = cb_first;
  while (true) {
#pragma unroll
    for (int s = 0; s < DE; ++s)
      if (R.b[s].cb >= 0) exp_finish<RB>(a, F, lane, R.b[s]);
    cb += 4 * DE;
    if (cb >= cb_end) break;
    exp_ring_load<RB>(a, cb, cb_end, lane, R);
  }
}

// ---------------------------------------------------------------------------
// Cross-workgroup hand-off of split-K partial sums (see item_shrink and
// item_expand_wait). LORA_XWG selects the protocol:
//  1: every thread fences at agent scope (release before, acquire after).
//  2: one thread per workgroup fences, ordered with the others by barriers.
//  3: partials move with agent-scope (cache-coherent) accesses and the
//     counters with atomics; no cache-wide writeback or invalidate.
// ---------------------------------------------------------------------------
#ifndef LORA_XWG
#define LORA_XWG 3
#endif

// Returns a value that depends on the store having been performed (protocol
// 3 uses a returning atomic swap; the caller folds the results into LDS so
// the wave waits for every swap before it reaches the barrier).
__device__ __forceinline__ float xwg_store(float* p, float v) {
#if LORA_XWG == 3
  return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#else
  *p = v;
  return 0.f;
#endif
}
__device__ __forceinline__ float xwg_load(const float* p) {
#if LORA_XWG == 3
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#else
  return *p;
#endif
}
// Called by every thread after its partial stores; thread 0 increments *ctr
// and gets the previous value (other threads get 0).
__device__ __forceinline__ int xwg_signal(int* ctr) {
  int old = 0;
#if LORA_XWG == 1
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
#elif LORA_XWG == 2
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#else
  __syncthreads();
  if (threadIdx.x == 0) old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#endif
  return old;
}
// Thread 0 has seen the counter complete; make the partials visible to the
// whole workgroup (ends with a barrier).
__device__ __forceinline__ void xwg_acquire() {
#if LORA_XWG == 2
  if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
#elif LORA_XWG == 1
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#else
  __syncthreads();
#endif
}

// ---------------------------------------------------------------------------
// Items
// ---------------------------------------------------------------------------
struct Smem {
  float red[4 * 16 * 64];
  float Pl[kTileM * kLdp];
  TileInfo ti;
  int flag;
};

// X rows of the tile as a buffer resource: based at the tile's first row when
// rows are contiguous, at X itself for a token_rows gather.
template <typename PT>
__device__ __forceinline__ void tile_rows(const uint16_t* base, int64_t ld, int width, const PT& P,
                                          const TileInfo& t, __amdgpu_buffer_rsrc_t& r, uint32_t& off) {
  const int n = threadIdx.x & 31;
  const bool valid = n < t.cnt;
  if (P.token_rows) {
    r = mk_rsrc(base, (int64_t)0x7ffffff0);
    off = valid ? (uint32_t)((int64_t)P.token_rows[t.p0 + n] * ld * 2) : kOff;
  } else {
    r = mk_rsrc(base + (int64_t)t.p0 * ld, ((int64_t)(t.cnt - 1) * ld + width) * 2);
    off = valid ? (uint32_t)((int64_t)n * ld * 2) : kOff;
  }
}

template <int RB, typename PT>
__device__ __forceinline__ void shrink_range(const PT& P, const TileInfo& t, int kb, int ke,
                                             int wave, int lane, f32x16 (&acc)[RB]) {
  __amdgpu_buffer_rsrc_t xr;
  uint32_t xoff;
  tile_rows(P.X, P.ldx, P.K, P, t, xr, xoff);
#pragma unroll
  for (int b = 0; b < RB; ++b) acc[b] = zero_acc16();
  shrink_acc<RB>(xr, xoff, w_ptr(P, t), P.K, t.rank, kb, ke, wave, lane, acc);
}

// Writes Pl rows 0..31, columns < 32*RB (zero where rank/token invalid) to U.
template <typename PT>
__device__ __forceinline__ void store_u_from_lds(const PT& P, const TileInfo& t,
                                                 const float* Pl) {
  for (int e = threadIdx.x; e < kTileM * t.rank; e += kThreads) {
    const int n = e / t.rank, k = e - n * t.rank;
    if (n < t.cnt) P.U[(int64_t)(t.p0 + n) * P.ldu + k] = Pl[n * kLdp + k];
  }
}

template <typename PT>
__device__ __forceinline__ ExpArgs exp_args(const PT& P, const TileInfo& t) {
  ExpArgs a;
  tile_rows(P.Y, P.ldy, P.N, P, t, a.yr, a.yoff);
  a.ldv = ((t.rank + P.v_round - 1) / P.v_round) * P.v_round;
  a.vec16 = (a.ldv & 7) == 0;
  a.vr = mk_rsrc(v_ptr(P, t), (int64_t)P.N * a.ldv * 2);
  a.rank = t.rank;
  a.ncols = P.N;
  a.oscale = P.scale_in_shrink ? 1.f : t.scale;
  return a;
}

// Column-block range of n-chunk c: this wave starts at cb0 + wave.
template <typename PT>
__device__ __forceinline__ void chunk_blocks(const PT& P, int c, int& cb0, int& cb_end) {
  const int nblocks = (P.N + 31) >> 5;
  cb0 = c * P.nblk;
  cb_end = min(nblocks, cb0 + P.nblk);
}

template <int RB, typename PT>
__device__ __forceinline__ void expand_tile_from_lds(const PT& P, const TileInfo& t, int c,
                                                     const float* Pl, int wave, int lane) {
  const ExpArgs a = exp_args(P, t);
  int cb0, cb_end;
  chunk_blocks(P, c, cb0, cb_end);
  ExpRing<RB> R;
  exp_ring_load<RB>(a, cb0 + wave, cb_end, lane, R);
  PFrags<RB> F;
  build_pfrags<RB>(Pl, t.rank, lane, F);
  exp_ring_run<RB>(a, F, cb0 + wave, cb_end, lane, R);
}

// kModeFusedTile: full shrink of one tile on chip, then its n-chunk c.
template <int RB, typename PT>
__device__ __forceinline__ void item_fused_tile(const PT& P, Smem& S, const TileInfo& t, int c) {
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
template <int RB, typename PT>
__device__ __forceinline__ void item_expand(const PT& P, Smem& S, const TileInfo& t, int c) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* Pl = S.Pl;
  for (int e = threadIdx.x; e < kTileM * 32 * RB; e += kThreads) {
    const int n = e / (32 * RB), k = e - n * (32 * RB);
    Pl[n * kLdp + k] = (n < t.cnt && k < t.rank) ? P.U[(int64_t)(t.p0 + n) * P.ldu + k] : 0.f;
  }
  __syncthreads();
  expand_tile_from_lds<RB>(P, t, c, Pl, wave, lane);
}

template <typename PT>
__device__ __forceinline__ float* partial_ptr(const PT& P, int g, int c) {
  return P.partials + ((int64_t)g * P.ks + c) * kTileM * P.rpad;
}

// kModeShrink / kModeFusedDep phase A: shrink over k-chunk c.
template <int RB, typename PT>
__device__ __forceinline__ void item_shrink(const PT& P, Smem& S, const TileInfo& t, int c) {
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
  float sink = 0.f;
  reduce_waves<RB>(S.red, acc, wave, lane,
                   [&](int k, int n, float v) { sink += xwg_store(part + n * rpad + k, v); });
#if LORA_XWG == 3
  S.red[threadIdx.x] = sink;  // waits for every swap of this thread
#else
  (void)sink;
#endif
  int* ctr = P.counters + kCtrTiles + t.g;
  const int old = xwg_signal(ctr);
  // storing the returned count makes thread 0 wait for its increment to be
  // performed before anything later (e.g. the done count) is issued
  if (threadIdx.x == 0) S.flag = old;
  if (P.mode == kModeFusedDep) return;
  // kModeShrink, ks > 1: the last arriving chunk sums all chunks in order
  __syncthreads();
  if (S.flag != P.ks - 1) return;
  xwg_acquire();
  for (int e = threadIdx.x; e < kTileM * t.rank; e += kThreads) {
    const int n = e / t.rank, k = e - n * t.rank;
    if (n >= t.cnt) continue;
    float s = xwg_load(partial_ptr(P, t.g, 0) + n * rpad + k);
    for (int q = 1; q < P.ks; ++q) s += xwg_load(partial_ptr(P, t.g, q) + n * rpad + k);
    P.U[(int64_t)(t.p0 + n) * P.ldu + k] = s * ps;
  }
  if (threadIdx.x == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// kModeFusedDep phase B: wait for the tile's k-chunks, sum them, expand.
// If the chunks do not arrive within spin_ticks (e.g. their workgroups are
// not resident), the item computes the same chunks itself in the same order,
// so the result is identical and no wait is unbounded.
template <int RB, typename PT>
__device__ __forceinline__ void item_expand_wait(const PT& P, Smem& S, const TileInfo& t, int c) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int* ctr = P.counters + kCtrTiles + t.g;
  // the y rows and expand weights do not depend on the shrink: load the
  // first block before waiting
  const ExpArgs ea = exp_args(P, t);
  int cb0, cb_end;
  chunk_blocks(P, c, cb0, cb_end);
  ExpRing<RB> R;
  exp_ring_load<RB>(ea, cb0 + wave, cb_end, lane, R);
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
  xwg_acquire();
  const float ps = P.scale_in_shrink ? t.scale : 1.f;
  float* Pl = S.Pl;
  const int rcols = 32 * RB;
  if (S.flag) {
    const int rpad = P.rpad;
    for (int e = threadIdx.x; e < kTileM * rcols; e += kThreads) {
      const int n = e / rcols, k = e - n * rcols;
      float s = xwg_load(partial_ptr(P, t.g, 0) + n * rpad + k);
      for (int q = 1; q < P.ks; ++q) s += xwg_load(partial_ptr(P, t.g, q) + n * rpad + k);
      Pl[n * kLdp + k] = s * ps;
    }
  } else {
    // the prefetched blocks are dropped while the shrink is recomputed
    // (keeps both register sets from being live at once) and loaded again
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
    exp_ring_load<RB>(ea, cb0 + wave, cb_end, lane, R);
  }
  __syncthreads();
  if (P.write_u && c == 0) store_u_from_lds(P, t, Pl);
  PFrags<RB> F;
  build_pfrags<RB>(Pl, t.rank, lane, F);
  exp_ring_run<RB>(ea, F, cb0 + wave, cb_end, lane, R);
}

template <int RB, typename PT>
__device__ __forceinline__ void run_item(const PT& P, Smem& S, const TileInfo& t, int kind, int c) {
  switch (kind) {
    case 0: item_shrink<RB>(P, S, t, c); break;
    case 1: item_expand<RB>(P, S, t, c); break;
    case 2: item_fused_tile<RB>(P, S, t, c); break;
    default: item_expand_wait<RB>(P, S, t, c); break;
  }
}

template <int RBMAX, typename PT>
__global__ __launch_bounds__(kThreads) void sgmv_fwd_kernel(PT P) {
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
    const TileInfo t = tile_info(P, g, &S.ti);
    if (RBMAX == 1 || t.rank <= 32) run_item<1>(P, S, t, kind, c);
    else if (RBMAX == 2 || t.rank <= 64) run_item<(RBMAX >= 2 ? 2 : 1)>(P, S, t, kind, c);
    else run_item<RBMAX>(P, S, t, kind, c);
  }
  if (P.mode == kModeFusedDep) {
    // the last workgroup to finish returns every counter of this launch to
    // zero (thread 0's earlier counter atomics have returned before this one
    // is issued, so every tile increment lands before the done count does)
    __syncthreads();
    if (threadIdx.x == 0) {
      const int old = __hip_atomic_fetch_add(P.counters + kCtrDone, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      if (old == P.grid - 1) {
        for (int g = 0; g < P.n_tiles; ++g)
          __hip_atomic_store(P.counters + kCtrTiles + g, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(P.counters + kCtrDone, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

template <typename PT>
static hipError_t launch_fwd_t(const PT& P, int rbmax, hipStream_t stream) {
  if (rbmax <= 1)
    hipLaunchKernelGGL((sgmv_fwd_kernel<1, PT>), dim3(P.grid), dim3(kThreads), 0, stream, P);
  else if (rbmax == 2)
    hipLaunchKernelGGL((sgmv_fwd_kernel<2, PT>), dim3(P.grid), dim3(kThreads), 0, stream, P);
  else
    hipLaunchKernelGGL((sgmv_fwd_kernel<4, PT>), dim3(P.grid), dim3(kThreads), 0, stream, P);
  return hipGetLastError();
}

// Launches with the smallest plan type that holds the segments: the plan is
// the kernel argument, and its size is part of every launch's host cost.
hipError_t launch_fwd(const FwdPlan& P, int rbmax, hipStream_t stream) {
  if (P.n_seg <= kSmallSeg) {
    FwdPlanT<kSmallSeg> Q;
    static_cast<FwdHeader&>(Q) = static_cast<const FwdHeader&>(P);
    for (int i = 0; i < P.n_seg; ++i) {
      Q.seg_tok0[i] = P.seg_tok0[i];
      Q.seg_ntok[i] = P.seg_ntok[i];
      Q.seg_tile0[i] = P.seg_tile0[i];
      Q.seg_adapter[i] = P.seg_adapter[i];
      Q.seg_scale[i] = P.seg_scale[i];
      Q.seg_rank[i] = P.seg_rank[i];
      Q.seg_slot[i] = P.seg_slot[i];
    }
    return launch_fwd_t(Q, rbmax, stream);
  }
  return launch_fwd_t(P, rbmax, stream);
}

}  // namespace lora
