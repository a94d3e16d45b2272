// lora_fwd.hip -- shrink / expand / fused multi-adapter LoRA kernels for gfx950.
//
// Method: every token of a batch carries an adapter; the batch is cut into
// segments of one adapter each and a single launch covers all of them
// ("Trajectory presenta C-LoRA" (vivodigitale.it), "Come funziona
// l'architettura"). Work is tiled along the token (sequence) and hidden
// dimensions, never along the small rank ("Technische Samenvatting: PLoRA"
// (gist.science), "Kernelontwerp"). The same kernel serves the backward du/dx
// pass with dy in place of x, B^T in place of A and A^T in place of B.
//
// One workgroup (4 wave64) owns a tile of 32 tokens of one segment:
//  shrink  P^T[rank][token] += W[rank][k] * X[token][k]
//  expand  Y^T[col][token]  += V[col][rank] * P^T[rank][token]
// both on v_mfma_f32_32x32x16_bf16 with fp32 accumulation; fp32 P enters the
// expand as a bf16 hi + lo pair. Global memory is touched only with
// row-contiguous 16-byte accesses (consecutive lanes take consecutive 16
// bytes of a row): chunks of X, W, y and V are staged through padded LDS rows
// and the MFMA operands are read from LDS. The next chunk's global loads are
// issued before the current chunk is computed.
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

template <typename PT>
struct PlanCap;
template <int CAP>
struct PlanCap<FwdPlanT<CAP>> {
  static constexpr int v = CAP;  // segment capacity of a plan type
};

// Finds the segment that holds tile g. Small plans (decode batches): a scalar
// scan of the whole table, which the compiler reads from the kernel
// arguments with a few wide scalar loads, with no LDS round trip or barrier.
// Large plans: one parallel read of the table (thread i checks segment i and
// the matching thread publishes the tile's description in LDS).
template <typename PT>
__device__ __forceinline__ TileInfo tile_info(const PT& P, int g, TileInfo* lds) {
  constexpr int CAP = PlanCap<PT>::v;
  if constexpr (CAP <= kSmallSeg) {
    int sel = 0;
#pragma unroll
    for (int i = 1; i < CAP; ++i)
      if (i < P.n_seg && g >= P.seg_tile0[i]) sel = i;
    TileInfo t;
    const int tt = g - P.seg_tile0[sel];
    t.g = g;
    t.p0 = P.seg_tok0[sel] + tt * kTileM;
    t.cnt = min(kTileM, P.seg_ntok[sel] - tt * kTileM);
    t.adapter = P.seg_adapter[sel];
    t.rank = P.seg_rank[sel];
    t.slot = P.seg_slot[sel];
    t.scale = P.seg_scale[sel];
    return t;
  }
  // the table reads do not wait for n_seg: entries past it are in the plan
  // too, and only the comparison uses n_seg
  const int i = min((int)threadIdx.x, PlanCap<PT>::v - 1);
  const int t0 = P.seg_tile0[i];
  const int t1n = P.seg_tile0[min(i + 1, PlanCap<PT>::v - 1)];
  const int tok0 = P.seg_tok0[i], ntok = P.seg_ntok[i];
  const int adapter = P.seg_adapter[i], rank = P.seg_rank[i], slot = P.seg_slot[i];
  const float scale = P.seg_scale[i];
  if (threadIdx.x < P.n_seg) {
    const int t1 = (i + 1 < P.n_seg) ? t1n : P.n_tiles;
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

// Workgroup barrier for LDS hand-offs between waves. Global loads that are in
// flight across it belong to the calling wave only and are waited for where
// their registers are used.
__device__ __forceinline__ void lds_sync() { __syncthreads(); }

// ---------------------------------------------------------------------------
// Chunk geometry for RB 32-row rank blocks (rank <= 32 * RB).
//
// Shrink chunks are loaded straight into LDS, one 1 KB block per wave
// instruction (lane l's 16 bytes land at block + 16 l). A block holds R whole
// rows of the chunk (KC elements each); the block stride is padded by R
// 16-byte slots, and slot (row q of the block, 16-byte column c) is
// SR q + (c ^ q): the 32 rows of an MFMA fragment then fall on distinct
// bank groups, and every instruction still reads whole rows from memory.
// ---------------------------------------------------------------------------
template <int RB>
struct Geo {
  static constexpr int KC = RB == 1 ? 256 : (RB == 2 ? 128 : 64);  // shrink k-chunk (elements)
  static constexpr int R = 1024 / (2 * KC);                       // rows per LDS block
  static constexpr int SR = 64 / R;                               // 16-byte slots per row
  static constexpr int BS = 1024 + 16 * R;                        // LDS block stride (bytes)
  static constexpr int NBX = 32 / R;                              // blocks of X rows
  static constexpr int NBW = 32 * RB / R;                         // blocks of W rows
  static constexpr int BPW = (NBX + NBW) / 4;                     // block loads per wave
  static constexpr int SHRINK_BYTES = (NBX + NBW) * BS;
  static constexpr int CW = RB == 1 ? 256 : 128;                  // expand column chunk
  static constexpr int CWP = CW + 8;                              // LDS row of y (elements)
  static constexpr int RP = 32 * RB + 8;                          // LDS row of V (elements)
  static constexpr int YV = (32 * CW / 8) / kThreads;             // y vectors per thread
  static constexpr int VV = (CW * 4 * RB) / kThreads;             // V vectors per thread (at most)
  static constexpr int EXPAND_BYTES = 32 * CWP * 2 + CW * RP * 2;
  static_assert(NBX % 4 == 0 && NBW % 4 == 0, "block loads split evenly over the waves");
};

constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int kRedBytes = 4 * 16 * 64 * 4;             // wave-reduction buffer
constexpr int kPlBytes = kTileM * kLdp * 4;             // the tile's P (fp32)
template <int RBMAX>
struct LdsBytes {
  static constexpr int shrink = cmax(Geo<1>::SHRINK_BYTES, cmax(RBMAX >= 2 ? Geo<2>::SHRINK_BYTES : 0,
                                                                RBMAX >= 4 ? Geo<4>::SHRINK_BYTES : 0));
  static constexpr int expand = cmax(Geo<1>::EXPAND_BYTES, cmax(RBMAX >= 2 ? Geo<2>::EXPAND_BYTES : 0,
                                                                RBMAX >= 4 ? Geo<4>::EXPAND_BYTES : 0));
  // buffer 0: shrink chunks, the wave reduction, the expand stage
  static constexpr int b0 = cmax(shrink, cmax(expand, kRedBytes));
  // buffer 1: shrink chunks, the tile's P
  static constexpr int b1 = cmax(shrink, kPlBytes);
};

// The workgroup's LDS. The two buffers are separate arrays so that the
// compiler can tell loads into one from reads of the other.
struct Lds {
  uint8_t* b0;
  uint8_t* b1;
  TileInfo* ti;
  int* flag;
  __device__ float* Pl() const { return reinterpret_cast<float*>(b1); }
  __device__ float* red() const { return reinterpret_cast<float*>(b0); }
};

// Rows of a tile as a buffer resource: based at the tile's first row when
// rows are contiguous, at the matrix itself for a token_rows gather.
struct TileRows {
  __amdgpu_buffer_rsrc_t r;
  int64_t ld2;  // row stride in bytes
  bool gather;
};
template <typename PT>
__device__ __forceinline__ TileRows tile_rows(const uint16_t* base, int64_t ld, int width, const PT& P,
                                              const TileInfo& t) {
  TileRows tr;
  tr.gather = P.token_rows != nullptr;
  tr.ld2 = ld * 2;
  if (tr.gather)
    tr.r = mk_rsrc(base, (int64_t)0x7ffffff0);
  else
    tr.r = mk_rsrc(base + (int64_t)t.p0 * ld, ((int64_t)(t.cnt - 1) * ld + width) * 2);
  return tr;
}
// Byte offset of tile row n in the resource (kOff if not a valid token).
template <typename PT>
__device__ __forceinline__ uint32_t row_off(const PT& P, const TileInfo& t, const TileRows& tr, int n) {
  if (n >= t.cnt) return kOff;
  const int64_t row = tr.gather ? (int64_t)P.token_rows[t.p0 + n] : (int64_t)n;
  return (uint32_t)(row * tr.ld2);
}

// ---------------------------------------------------------------------------
// Shrink over k in [kb, ke). Chunk c covers KC columns of the tile's 32 X rows
// and of the 32*RB W rows; rows past the tile or the rank, and columns past
// ke, land in LDS as zeros (out-of-range buffer lanes write zeros). Wave w
// loads blocks w, w+4, ...; the 4 waves then split the chunk's k-steps and
// read MFMA fragments from LDS; acc[b] holds P^T rows 32b.. of the wave's
// partial sum. Chunks alternate between the two LDS buffers, so chunk c+1 is
// in flight while chunk c is computed.
// ---------------------------------------------------------------------------
// s_waitcnt immediates (gfx9 encoding): vmcnt(n) alone, lgkmcnt(0) alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier without the memory fence of __syncthreads: the caller
// waits for exactly the memory operations the other waves depend on.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int RB>
struct ShrinkCtx {
  i32x4 xr, wr;
  uint32_t roff[Geo<RB>::BPW];  // byte offset of this lane's row in each of the wave's blocks
  uint32_t cbytes;              // this lane's column within a chunk (bytes)
  int kb, ke;
};

// Issues the wave's block loads of chunk `chunk` into `buf`.
template <int RB>
__device__ __forceinline__ void shrink_issue(const ShrinkCtx<RB>& C, int chunk, uint8_t* buf, int wave) {
  using G = Geo<RB>;
  const int k0 = C.kb + chunk * G::KC;
  const int k = k0 + (int)(C.cbytes >> 1);
  const bool kv = k < C.ke;
  const uint32_t kbytes = 2u * (uint32_t)k0 + C.cbytes;
  // block wave + 4 j; NBX is a multiple of 4, so j < NBX / 4 are the X blocks.
  // The LDS destination must be scalar (it goes to M0).
  const uint32_t base = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)((uint32_t)reinterpret_cast<uintptr_t>(buf) + (uint32_t)wave * G::BS));
#pragma unroll
  for (int j = 0; j < G::NBX / 4; ++j) load_lds16(C.xr, base + 4u * j * G::BS, kv ? C.roff[j] + kbytes : kOff);
#pragma unroll
  for (int j = G::NBX / 4; j < G::BPW; ++j)
    load_lds16(C.wr, base + 4u * j * G::BS, kv ? C.roff[j] + kbytes : kOff);
}

// Byte offset in a chunk buffer of 16-byte column c of row `row` of the x
// (w = false) or W (w = true) rows.
template <int RB>
__device__ __forceinline__ uint32_t slot_off(int row, int c, bool w) {
  using G = Geo<RB>;
  const int q = row % G::R;
  return (uint32_t)(((w ? G::NBX : 0) + row / G::R) * G::BS + 16 * (G::SR * q + (c ^ q)));
}

template <int RB>
__device__ __forceinline__ void shrink_mfma(const uint8_t* buf, int wave, int lane, f32x16 (&acc)[RB]) {
  using G = Geo<RB>;
  constexpr int SPW = G::KC / 64;  // k-steps of 16 per wave per chunk
  const int h = lane >> 5, m = lane & 31;
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int c = 2 * (wave * SPW + s) + h;
    const u32x4 xf = ld16(buf + slot_off<RB>(m, c, false));
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const u32x4 wf = ld16(buf + slot_off<RB>(32 * b + m, c, true));
      acc[b] = mfma32(as_bf16x8(wf), as_bf16x8(xf), acc[b]);
    }
  }
}

template <int RB, typename PT>
__device__ __forceinline__ void shrink_lds(const PT& P, const TileInfo& t, int kb, int ke, const Lds& L,
                                           f32x16 (&acc)[RB]) {
  using G = Geo<RB>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // lane -> (row q of the block, 16-byte column c): slot lane = SR q + (c ^ q)
  const int q = lane / G::SR;
  const int c = (lane % G::SR) ^ q;
  ShrinkCtx<RB> C;
  const TileRows xt = tile_rows(P.X, P.ldx, P.K, P, t);
  if (xt.gather)
    C.xr = mk_rsrc_words(P.X, (int64_t)0x7ffffff0);
  else
    C.xr = mk_rsrc_words(P.X + (int64_t)t.p0 * P.ldx, ((int64_t)(t.cnt - 1) * P.ldx + P.K) * 2);
  const uint32_t ldw2 = 2u * (uint32_t)P.K;
  C.wr = mk_rsrc_words(w_ptr(P, t), (int64_t)t.rank * ldw2);  // rows >= rank fall outside
#pragma unroll
  for (int j = 0; j < G::BPW; ++j) {
    const int blk = wave + 4 * j;
    C.roff[j] = j < G::NBX / 4 ? row_off(P, t, xt, G::R * blk + q) : (uint32_t)(G::R * (blk - G::NBX) + q) * ldw2;
  }
  C.cbytes = 16u * (uint32_t)c;
  C.kb = kb;
  C.ke = ke;
#pragma unroll
  for (int b = 0; b < RB; ++b) acc[b] = zero_acc16();
  const int nch = __builtin_amdgcn_readfirstlane((ke - kb + G::KC - 1) / G::KC);
  if (nch <= 0) return;
  // every wave's loads of a chunk must have landed before any wave reads it:
  // wait for this wave's loads of the chunk (its later chunk may stay in
  // flight), then barrier. Before a buffer is loaded again, every wave's
  // reads of it must be done: wait for LDS reads, then barrier.
  auto step = [&](uint8_t* buf, int cc) {
    if (cc + 1 < nch)
      wait_vmcnt<G::BPW>();
    else
      wait_vmcnt<0>();
    raw_barrier();
    shrink_mfma<RB>(buf, wave, lane, acc);
    wait_lgkmcnt0();
    raw_barrier();
    if (cc + 2 < nch) shrink_issue<RB>(C, cc + 2, buf, wave);
  };
  shrink_issue<RB>(C, 0, L.b0, wave);
  shrink_issue<RB>(C, 1, L.b1, wave);  // past the range: zeros, waited for below
  for (int cc = 0; cc < nch; cc += 2) {
    step(L.b0, cc);
    if (cc + 1 >= nch) break;
    step(L.b1, cc + 1);
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
    lds_sync();
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
    lds_sync();
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
// P[token = lane%32][16kb + 8(lane/32) + e], zero for k >= rank.
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

// Expand of the item's columns [c0, c1) in chunks of CW columns. A chunk's
// 32 y rows and its CW rows of V (one contiguous span of V) are staged
// through LDS; every wave computes whole 32-column blocks from LDS, with the
// rows of a block permuted by colmap so that a lane owns two runs of 8
// contiguous bf16 of one y row; the results go back into the LDS y tile,
// which is then stored row-contiguously.
template <int RB>
struct ExpRegs {
  u32x4 y[Geo<RB>::YV];
  u32x4 v[Geo<RB>::VV];
};

template <int RB>
struct ExpCtx {
  __amdgpu_buffer_rsrc_t yr, vr;
  uint32_t yoff[Geo<RB>::YV];  // byte offset of this thread's y rows
  uint16_t vrow[Geo<RB>::VV];  // V vector f = t + 256j of a chunk: row within the chunk
  uint16_t vlds[Geo<RB>::VV];  // and its element offset in the LDS V tile
  int64_t ldv;                 // V row stride (elements)
  int rank, kbn;               // rank, k-steps of 16 that hold rank columns
  int nv;                      // 16-byte V vectors per chunk (vec16)
  bool vec16;                  // V rows are whole 16-byte vectors
  int c0, c1;                  // column range of the item
  float oscale;
};

template <int RB>
__device__ __forceinline__ void exp_load(const ExpCtx<RB>& C, int cs, ExpRegs<RB>& R) {
  using G = Geo<RB>;
  constexpr int YPR = G::CW / 8;
  const int col = cs + 8 * (threadIdx.x % YPR);
  const bool cv = col < C.c1;
  const uint32_t cbytes = 2u * (uint32_t)col;
#pragma unroll
  for (int j = 0; j < G::YV; ++j) R.y[j] = bld16(C.yr, cv ? C.yoff[j] + cbytes : kOff);
  if (C.vec16) {
    // the chunk's V rows [cs, cs + CW) are one contiguous span
    const uint32_t base = (uint32_t)(cs * C.ldv * 2);
#pragma unroll
    for (int j = 0; j < G::VV; ++j) {
      const int f = threadIdx.x + kThreads * j;
      const bool ok = f < C.nv && cs + C.vrow[j] < C.c1;
      R.v[j] = bld16(C.vr, ok ? base + 16u * (uint32_t)f : kOff);
    }
  }
}

template <int RB>
__device__ __forceinline__ void exp_to_lds(const ExpCtx<RB>& C, int cs, const ExpRegs<RB>& R,
                                           uint16_t* ys, uint16_t* vs) {
  using G = Geo<RB>;
  constexpr int YPR = G::CW / 8;
  constexpr int RPJ = kThreads / YPR;
  const int r0 = threadIdx.x / YPR, c = 8 * (threadIdx.x % YPR);
#pragma unroll
  for (int j = 0; j < G::YV; ++j) st16(ys + (r0 + RPJ * j) * G::CWP + c, R.y[j]);
  if (C.vec16) {
#pragma unroll
    for (int j = 0; j < G::VV; ++j)
      if (threadIdx.x + kThreads * j < C.nv) st16(vs + C.vlds[j], R.v[j]);
  } else {
    // rows not made of whole 16-byte vectors: element loads straight to LDS
    const int kw = 16 * C.kbn;
    for (int e = threadIdx.x; e < G::CW * kw; e += kThreads) {
      const int row = e / kw, k = e - row * kw;
      const bool ok = k < C.rank && cs + row < C.c1;
      vs[row * G::RP + k] = (uint16_t)bld2(C.vr, ok ? (uint32_t)(((cs + row) * C.ldv + k) * 2) : kOff);
    }
  }
}

template <int RB>
__device__ __forceinline__ void exp_mfma(const ExpCtx<RB>& C, const PFrags<RB>& F, int cs, uint16_t* ys,
                                         const uint16_t* vs, int wave, int lane) {
  using G = Geo<RB>;
  constexpr int NB = G::CW / 32;  // 32-column blocks per chunk
  const int m = lane & 31, h = lane >> 5;
#pragma unroll
  for (int q = wave; q < NB; q += 4) {
    const int col0 = 32 * q;
    if (cs + col0 >= C.c1) break;  // uniform
    f32x16 acc = zero_acc16();
    const uint16_t* vrow = vs + (col0 + colmap(m)) * G::RP + 8 * h;
#pragma unroll
    for (int kb = 0; kb < 2 * RB; ++kb) {
      if (kb < C.kbn) {
        const u32x4 vf = ld16(vrow + 16 * kb);
        acc = mfma32(as_bf16x8(vf), F.hi[kb], acc);
        acc = mfma32(as_bf16x8(vf), F.lo[kb], acc);
      }
    }
    // token m, columns col0 + 8h + [0, 8) and col0 + 16 + 8h + [0, 8)
    uint16_t* yr = ys + m * G::CWP + col0 + 8 * h;
    float f[8];
    unpack8(ld16(yr), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = f[i] + C.oscale * acc[i];
    st16(yr, pack8(f));
    unpack8(ld16(yr + 16), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = f[i] + C.oscale * acc[8 + i];
    st16(yr + 16, pack8(f));
  }
}

template <int RB>
__device__ __forceinline__ void exp_store(const ExpCtx<RB>& C, int cs, const uint16_t* ys) {
  using G = Geo<RB>;
  constexpr int YPR = G::CW / 8;
  constexpr int RPJ = kThreads / YPR;
  const int r0 = threadIdx.x / YPR, c = 8 * (threadIdx.x % YPR);
  const int col = cs + c;
  const bool cv = col < C.c1;
  const uint32_t cbytes = 2u * (uint32_t)col;
#pragma unroll
  for (int j = 0; j < G::YV; ++j)
    bst16(C.yr, cv ? C.yoff[j] + cbytes : kOff, ld16(ys + (r0 + RPJ * j) * G::CWP + c));
}

template <int RB, typename PT>
__device__ __forceinline__ ExpCtx<RB> exp_ctx(const PT& P, const TileInfo& t, int c) {
  using G = Geo<RB>;
  constexpr int YPR = G::CW / 8;
  constexpr int RPJ = kThreads / YPR;
  ExpCtx<RB> C;
  const TileRows yt = tile_rows(P.Y, P.ldy, P.N, P, t);
  C.yr = yt.r;
  const int r0 = threadIdx.x / YPR;
#pragma unroll
  for (int j = 0; j < G::YV; ++j) C.yoff[j] = row_off(P, t, yt, r0 + RPJ * j);
  C.ldv = ((t.rank + P.v_round - 1) / P.v_round) * P.v_round;
  C.vec16 = (C.ldv & 7) == 0;
  C.vr = mk_rsrc(v_ptr(P, t), (int64_t)P.N * C.ldv * 2);
  C.rank = t.rank;
  C.kbn = (t.rank + 15) >> 4;
  const int rv = (int)(C.ldv >> 3);  // vectors per V row (vec16)
  C.nv = G::CW * rv;
  const float inv = 1.0f / (float)max(rv, 1);
#pragma unroll
  for (int j = 0; j < G::VV; ++j) {
    // row = f / rv exactly: (f + 0.5) / rv is at least 1/(2 rv) away from an integer
    const int f = threadIdx.x + kThreads * j;
    const int row = (int)(((float)f + 0.5f) * inv);
    C.vrow[j] = (uint16_t)row;
    C.vlds[j] = (uint16_t)(row * G::RP + 8 * (f - row * rv));
  }
  const int nblocks = (P.N + 31) >> 5;
  const int cb0 = c * P.nblk;
  C.c0 = 32 * cb0;
  C.c1 = min(P.N, 32 * min(nblocks, cb0 + P.nblk));
  C.oscale = P.scale_in_shrink ? 1.f : t.scale;
  return C;
}

// Chunks of the expand whose loads are in flight (register sets).
template <int RB>
struct ExpDepth {
  static constexpr int v = RB <= 2 ? 2 : 1;
};

// Runs the expand over the item's columns. R holds the loads of the first NE
// chunks, issued by the caller (so they can be issued before a wait).
template <int RB, int NE>
__device__ __forceinline__ void expand_run(const ExpCtx<RB>& C, const PFrags<RB>& F, ExpRegs<RB> (&R)[NE],
                                           uint8_t* stage) {
  using G = Geo<RB>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint16_t* ys = reinterpret_cast<uint16_t*>(stage);
  uint16_t* vs = ys + 32 * G::CWP;
  // a rank that ends half-way through a 16-wide k-step: the other half of
  // the last step is zero in every V row (written once; chunks never touch it)
  if (C.vec16 && (C.ldv & 8) && threadIdx.x < G::CW)
    st16(vs + threadIdx.x * G::RP + C.ldv, zero16());
  auto chunk = [&](int cs, ExpRegs<RB>& Rq) {
    exp_to_lds<RB>(C, cs, Rq, ys, vs);
    lds_sync();
    exp_load<RB>(C, cs + NE * G::CW, Rq);  // past the range: reads nothing
    exp_mfma<RB>(C, F, cs, ys, vs, wave, lane);
    lds_sync();
    exp_store<RB>(C, cs, ys);
    lds_sync();
  };
  // the first chunk is peeled so that the loop is entered with the same
  // kinds of accesses pending as on its back edge (later loads, then stores)
  if (C.c0 >= C.c1) return;
  chunk(C.c0, R[0]);
  int cs = C.c0 + G::CW;
  if constexpr (NE == 1) {
    for (; cs < C.c1; cs += G::CW) chunk(cs, R[0]);
  } else {
    for (; cs + G::CW < C.c1; cs += 2 * G::CW) {
      chunk(cs, R[1]);
      chunk(cs + G::CW, R[0]);
    }
    if (cs < C.c1) chunk(cs, R[1]);
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
// Writes Pl rows 0..cnt-1, columns < rank to U.
template <typename PT>
__device__ __forceinline__ void store_u_from_lds(const PT& P, const TileInfo& t, const float* Pl) {
  for (int e = threadIdx.x; e < kTileM * t.rank; e += kThreads) {
    const int n = e / t.rank, k = e - n * t.rank;
    if (n < t.cnt) P.U[(int64_t)(t.p0 + n) * P.ldu + k] = Pl[n * kLdp + k];
  }
}

template <int RB, typename PT>
__device__ __forceinline__ void expand_from_lds(const PT& P, const TileInfo& t, int c, const float* Pl,
                                                uint8_t* stage) {
  const ExpCtx<RB> C = exp_ctx<RB>(P, t, c);
  constexpr int NE = ExpDepth<RB>::v;
  ExpRegs<RB> R[NE];
#pragma unroll
  for (int q = 0; q < NE; ++q) exp_load<RB>(C, C.c0 + q * Geo<RB>::CW, R[q]);  // empty ranges read nothing
  PFrags<RB> F;
  build_pfrags<RB>(Pl, t.rank, threadIdx.x & 63, F);
  expand_run<RB, NE>(C, F, R, stage);
}

// kModeFusedTile: full shrink of one tile on chip, then its n-chunk c.
template <int RB, typename PT>
__device__ __forceinline__ void item_fused_tile(const PT& P, const Lds& L, const TileInfo& t, int c) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  f32x16 acc[RB];
  shrink_lds<RB>(P, t, 0, P.K, L, acc);
  const float ps = P.scale_in_shrink ? t.scale : 1.f;
  float* Pl = L.Pl();
  reduce_waves<RB>(L.red(), acc, wave, lane, [&](int k, int n, float v) { Pl[n * kLdp + k] = v * ps; });
  if (P.write_u && c == 0) store_u_from_lds(P, t, Pl);
  expand_from_lds<RB>(P, t, c, Pl, L.b0);
}

// kModeExpand: U from memory, expand n-chunk c.
template <int RB, typename PT>
__device__ __forceinline__ void item_expand(const PT& P, const Lds& L, const TileInfo& t, int c) {
  float* Pl = L.Pl();
  for (int e = threadIdx.x; e < kTileM * 32 * RB; e += kThreads) {
    const int n = e / (32 * RB), k = e - n * (32 * RB);
    Pl[n * kLdp + k] = (n < t.cnt && k < t.rank) ? P.U[(int64_t)(t.p0 + n) * P.ldu + k] : 0.f;
  }
  lds_sync();
  expand_from_lds<RB>(P, t, c, Pl, L.b0);
}

template <typename PT>
__device__ __forceinline__ float* partial_ptr(const PT& P, int g, int c) {
  return P.partials + ((int64_t)g * P.ks + c) * kTileM * P.rpad;
}

// kModeShrink / kModeFusedDep phase A: shrink over k-chunk c.
template <int RB, typename PT>
__device__ __forceinline__ void item_shrink(const PT& P, const Lds& L, const TileInfo& t, int c) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kb = c * P.kchunk;
  const int ke = min(P.K, kb + P.kchunk);
  f32x16 acc[RB];
  shrink_lds<RB>(P, t, kb, ke, L, acc);
  float* red = L.red();
  const float ps = P.scale_in_shrink ? t.scale : 1.f;
  if (P.mode == kModeShrink && P.ks == 1) {
    reduce_waves<RB>(red, acc, wave, lane, [&](int k, int n, float v) {
      if (n < t.cnt && k < t.rank) P.U[(int64_t)(t.p0 + n) * P.ldu + k] = v * ps;
    });
    return;
  }
  float* part = partial_ptr(P, t.g, c);
  const int rpad = P.rpad;
  float sink = 0.f;
  reduce_waves<RB>(red, acc, wave, lane,
                   [&](int k, int n, float v) { sink += xwg_store(part + n * rpad + k, v); });
#if LORA_XWG == 3
  red[threadIdx.x] = sink;  // waits for every swap of this thread
#else
  (void)sink;
#endif
  int* ctr = P.counters + kCtrTiles + t.g;
  const int old = xwg_signal(ctr);
  // storing the returned count makes thread 0 wait for its increment to be
  // performed before anything later (e.g. the done count) is issued
  if (threadIdx.x == 0) *L.flag = old;
  if (P.mode == kModeFusedDep) return;
  // kModeShrink, ks > 1: the last arriving chunk sums all chunks in order
  __syncthreads();
  if (*L.flag != P.ks - 1) return;
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
__device__ __forceinline__ void item_expand_wait(const PT& P, const Lds& L, const TileInfo& t, int c) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int* ctr = P.counters + kCtrTiles + t.g;
  // y rows and expand weights do not depend on the shrink: issue the first
  // chunk's loads before waiting
  const ExpCtx<RB> C = exp_ctx<RB>(P, t, c);
  constexpr int NE = ExpDepth<RB>::v;
  ExpRegs<RB> R[NE];
#pragma unroll
  for (int q = 0; q < NE; ++q) exp_load<RB>(C, C.c0 + q * Geo<RB>::CW, R[q]);  // empty ranges read nothing
  if (threadIdx.x == 0) {
    const uint64_t t0 = wall_clock64();
    int ready = 0;
    while (true) {
      if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= P.ks) { ready = 1; break; }
      if (wall_clock64() - t0 > (uint64_t)P.spin_ticks) break;
      __builtin_amdgcn_s_sleep(1);
    }
    *L.flag = ready;
  }
  xwg_acquire();
  const float ps = P.scale_in_shrink ? t.scale : 1.f;
  float* Pl = L.Pl();
  const int rcols = 32 * RB;
  if (*L.flag) {
    const int rpad = P.rpad;
    for (int e = threadIdx.x; e < kTileM * rcols; e += kThreads) {
      const int n = e / rcols, k = e - n * rcols;
      float s = xwg_load(partial_ptr(P, t.g, 0) + n * rpad + k);
      for (int q = 1; q < P.ks; ++q) s += xwg_load(partial_ptr(P, t.g, q) + n * rpad + k);
      Pl[n * kLdp + k] = s * ps;
    }
    lds_sync();
    if (P.write_u && c == 0) store_u_from_lds(P, t, Pl);
    PFrags<RB> F;
    build_pfrags<RB>(Pl, t.rank, lane, F);
    expand_run<RB, NE>(C, F, R, L.b0);
    return;
  }
  // Fallback. The early loads are dropped and issued again after the shrink
  // (a separate expand, so that they are not held in registers through it).
  // The chunk sums run in registers (each thread always receives the same
  // elements from the reduction) because the shrink reuses P's LDS buffer;
  // the last chunk's pass writes P.
  float run[4 * RB];
  for (int q = 0; q < P.ks; ++q) {
    const int kb = q * P.kchunk;
    const int ke = min(P.K, kb + P.kchunk);
    f32x16 acc[RB];
    shrink_lds<RB>(P, t, kb, ke, L, acc);
    int idx = 0;
    const bool last = q == P.ks - 1;
    reduce_waves<RB>(L.red(), acc, wave, lane, [&](int k, int n, float v) {
      const float sum = (q == 0) ? v : run[idx] + v;
      run[idx] = sum;
      if (last) Pl[n * kLdp + k] = sum * ps;
      ++idx;
    });
  }
  lds_sync();
  if (P.write_u && c == 0) store_u_from_lds(P, t, Pl);
  expand_from_lds<RB>(P, t, c, Pl, L.b0);
}

template <int RB, typename PT>
__device__ __forceinline__ void run_item(const PT& P, const Lds& L, const TileInfo& t, int kind, int c) {
  switch (kind) {
    case 0: item_shrink<RB>(P, L, t, c); break;
    case 1: item_expand<RB>(P, L, t, c); break;
    case 2: item_fused_tile<RB>(P, L, t, c); break;
    default: item_expand_wait<RB>(P, L, t, c); break;
  }
}

template <int RBMAX, typename PT>
__global__ __launch_bounds__(kThreads, 2) void sgmv_fwd_kernel(PT P) {
  __shared__ alignas(16) uint8_t lds_b0[LdsBytes<RBMAX>::b0];
  __shared__ alignas(16) uint8_t lds_b1[LdsBytes<RBMAX>::b1];
  __shared__ TileInfo lds_ti;
  __shared__ int lds_flag;
  const Lds L{lds_b0, lds_b1, &lds_ti, &lds_flag};
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
    const TileInfo t = tile_info(P, g, L.ti);
    if (RBMAX == 1 || t.rank <= 32) run_item<1>(P, L, t, kind, c);
    else if (RBMAX == 2 || t.rank <= 64) run_item<(RBMAX >= 2 ? 2 : 1)>(P, L, t, kind, c);
    else run_item<RBMAX>(P, L, t, kind, c);
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
    FwdPlanT<kSmallSeg> Q{};
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
