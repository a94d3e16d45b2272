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
  int proj;  // projection (multi-projection launches; else 0)
  float scale;
  uint64_t wptr, vptr;  // small plans with ptrs_in_plan: the segment's weight addresses
  const int* rows;      // batches planned inside the launch: the tile's rows (LDS)
  uint64_t lid;         // ... the launch id of the split hand-off
  int nblk;             // ... and the 32-column blocks per expand chunk
};

template <typename PT>
struct PlanCap;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winvalid-offsetof"
template <int CAP>
struct PlanCap<FwdPlanT<CAP>> {
  static constexpr int v = CAP;  // segment capacity of a plan type
  static constexpr bool self = false;  // launches planned inside themselves
  static constexpr bool rows = false;  // plans that carry the token-row table
  // byte offsets of the weight-address arrays in the plan, which is the
  // kernel's only explicit argument and so starts the kernel-argument segment
  static constexpr int kOffW = __builtin_offsetof(FwdPlanT<CAP>, seg_wptr);
  static constexpr int kOffV = __builtin_offsetof(FwdPlanT<CAP>, seg_vptr);
  // and of the byte arrays, read as the 32-bit word that holds the entry
  static constexpr int kOffRank = __builtin_offsetof(FwdPlanT<CAP>, seg_rank);
  static constexpr int kOffSlot = __builtin_offsetof(FwdPlanT<CAP>, seg_slot);
  static constexpr int kOffProj = __builtin_offsetof(FwdPlanT<CAP>, seg_proj);
};
#pragma clang diagnostic pop
// The plan of launches planned inside themselves: the small plan's layout
// under a type of its own, so that they get kernel instances of their own
// and the code of every other launch is left as it is.
struct FwdPlanSelf : FwdPlanT<kSmallSeg> {};
template <>
struct PlanCap<FwdPlanSelf> : PlanCap<FwdPlanT<kSmallSeg>> {
  static constexpr bool self = true;
};
// A small plan that also carries the sorted-position -> row table (from the
// caller's host copy), so that a request-order batch needs no table in
// device memory and no upload before the launch.
struct FwdPlanRows : FwdPlanT<kSmallSeg> {
  int32_t rows[kPlanRows];
};
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winvalid-offsetof"
template <>
struct PlanCap<FwdPlanRows> : PlanCap<FwdPlanT<kSmallSeg>> {
  static constexpr bool rows = true;
  static constexpr int kOffRows = __builtin_offsetof(FwdPlanRows, rows);
};
#pragma clang diagnostic pop

// Finds the segment that holds tile g. Small plans (decode batches): a scalar
// scan of the whole table, which the compiler reads from the kernel
// arguments with a few wide scalar loads, with no LDS round trip or barrier.
// Large plans: one parallel read of the table (thread i checks segment i and
// the matching thread publishes the tile's description in LDS).
template <typename PT>
__device__ __forceinline__ TileInfo tile_info(const PT& P, int g, TileInfo* lds) {
  constexpr int CAP = PlanCap<PT>::v;
  if constexpr (CAP <= kSmallSeg) {
    if (P.dev_tiles) {
      // planned on the device: the plan kernel of this call wrote the tile
      // table before the launch (a tile past its count is empty)
      const int n = *P.dev_count;
      const DevTile* d = P.dev_tiles + g;
      TileInfo t;
      t.g = g;
      t.p0 = d->tok0;
      t.cnt = g < n ? d->cnt : 0;
      t.adapter = d->adapter;
      t.rank = d->rank;
      t.slot = 0;
      t.proj = 0;
      t.scale = d->scale;
      t.wptr = d->wptr;
      t.vptr = d->vptr;
      t.g = __builtin_amdgcn_readfirstlane(t.g);
      t.p0 = __builtin_amdgcn_readfirstlane(t.p0);
      t.cnt = __builtin_amdgcn_readfirstlane(t.cnt);
      t.adapter = __builtin_amdgcn_readfirstlane(t.adapter);
      t.rank = __builtin_amdgcn_readfirstlane(t.rank);
      t.scale = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, t.scale)));
      return t;
    }
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
    t.scale = P.seg_scale[sel];
    // one scalar load each from the kernel-argument segment at the selected
    // entry (indexing the arrays by value would hold all of them in SGPRs;
    // a byte entry indexed by value is otherwise read with a vector load)
    const auto* kb = (const char __attribute__((address_space(4)))*)__builtin_amdgcn_kernarg_segment_ptr();
    {
      static_assert(CAP % 4 == 0 && PlanCap<PT>::kOffRank % 4 == 0 && PlanCap<PT>::kOffSlot % 4 == 0 &&
                        PlanCap<PT>::kOffProj % 4 == 0,
                    "a byte entry's word lies inside its array");
      typedef const uint32_t __attribute__((address_space(4)))* KWord;
      const int word = sel & ~3, shift = 8 * (sel & 3);
      t.rank = (int)((*reinterpret_cast<KWord>(kb + PlanCap<PT>::kOffRank + word) >> shift) & 0xffu);
      t.slot = (int)((*reinterpret_cast<KWord>(kb + PlanCap<PT>::kOffSlot + word) >> shift) & 0xffu);
      t.proj = (int)((*reinterpret_cast<KWord>(kb + PlanCap<PT>::kOffProj + word) >> shift) & 0xffu);
    }
    t.wptr = t.vptr = 0;
    if (P.ptrs_in_plan) {
      typedef const uint64_t __attribute__((address_space(4)))* KPtr;
      t.wptr = *reinterpret_cast<KPtr>(kb + PlanCap<PT>::kOffW + sel * 8);
      t.vptr = *reinterpret_cast<KPtr>(kb + PlanCap<PT>::kOffV + sel * 8);
    }
    return t;
  }
  // the table reads do not wait for n_seg: entries past it are in the plan
  // too, and only the comparison uses n_seg
  const int i = min((int)threadIdx.x, PlanCap<PT>::v - 1);
  const int t0 = P.seg_tile0[i];
  const int t1n = P.seg_tile0[min(i + 1, PlanCap<PT>::v - 1)];
  const int tok0 = P.seg_tok0[i], ntok = P.seg_ntok[i];
  const int adapter = P.seg_adapter[i], rank = P.seg_rank[i], slot = P.seg_slot[i];
  const int proj = P.seg_proj[i];
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
      t.proj = proj;
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
  t.proj = __builtin_amdgcn_readfirstlane(t.proj);
  t.scale = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, t.scale)));
  return t;
}

// The output side of a tile's projection: rows, row stride, width, column
// blocks per expand item, and the weight tables (projection 0 is the plan's
// own fields; the others come from the plan's projection arrays, read with
// constant indices so that they stay scalar kernel-argument loads).
struct ProjView {
  uint16_t* Y;
  int64_t ldy;
  const uint64_t* Wtab;
  const uint64_t* Vtab;
  int N;
  int nblk;
};
template <typename PT>
__device__ __forceinline__ ProjView proj_view(const PT& P, int p) {
  ProjView v{P.Y, P.ldy, P.Wtab, P.Vtab, P.N, P.nblk};
#pragma unroll
  for (int q = 1; q < kMaxProj; ++q)
    if (p == q) v = ProjView{P.proj_Y[q], P.proj_ldy[q], P.proj_Wtab[q], P.proj_Vtab[q], P.proj_N[q], P.proj_nblk[q]};
  return v;
}

// 32-column blocks per expand chunk of the item's projection (launches
// planned inside themselves: the count their workgroups chose).
template <typename PT>
__device__ __forceinline__ int item_nblk(const PT& P, const TileInfo& t) {
  if constexpr (PlanCap<PT>::self) return t.nblk;
  return proj_view(P, t.proj).nblk;
}

template <typename PT>
__device__ __forceinline__ const uint16_t* w_ptr(const PT& P, const TileInfo& t) {
  if constexpr (PlanCap<PT>::v <= kSmallSeg)
    if (P.ptrs_in_plan) return reinterpret_cast<const uint16_t*>(t.wptr);
  const uint64_t* tab = proj_view(P, t.proj).Wtab;
  if (tab) return reinterpret_cast<const uint16_t*>(tab[t.adapter]);
  return P.Wslots + (int64_t)t.slot * P.w_slot_elems;
}
template <typename PT>
__device__ __forceinline__ const uint16_t* v_ptr(const PT& P, const TileInfo& t) {
  if constexpr (PlanCap<PT>::v <= kSmallSeg)
    if (P.ptrs_in_plan) return reinterpret_cast<const uint16_t*>(t.vptr);
  const uint64_t* tab = proj_view(P, t.proj).Vtab;
  if (tab) return reinterpret_cast<const uint16_t*>(tab[t.adapter]);
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
  static constexpr int CW = RB == 1 ? 256 : 128;                  // staged expand column chunk
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
  // buffer 0: shrink chunks, the wave reduction, the staged expand
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
  int* rows;      // [kTileM] rows of a tile planned inside the launch
  uint64_t* lid;  // its launch id
  __device__ float* Pl() const { return reinterpret_cast<float*>(b1); }
  __device__ float* red() const { return reinterpret_cast<float*>(b0); }
};

// Rows of a tile as a buffer resource: based at the tile's first row when
// rows are contiguous, at the matrix itself for a token_rows gather.
struct TileRows {
  __amdgpu_buffer_rsrc_t r;
  int64_t ld2;  // row stride in bytes
  int64_t lim;  // gather: largest row offset (bytes) whose whole row lies in the resource
  bool gather;
};
template <typename PT>
__device__ __forceinline__ TileRows tile_rows(const uint16_t* base, int64_t ld, int width, const PT& P,
                                              const TileInfo& t) {
  TileRows tr;
  tr.gather = PlanCap<PT>::self || PlanCap<PT>::rows || P.token_rows != nullptr;
  tr.ld2 = ld * 2;
  tr.lim = kGatherSpan - (int64_t)width * 2;
  if (tr.gather)
    tr.r = mk_rsrc(base, kGatherSpan);
  else
    tr.r = mk_rsrc(base + (int64_t)t.p0 * ld, ((int64_t)(t.cnt - 1) * ld + width) * 2);
  return tr;
}
// Byte offset of tile row n in the resource (kOff if not a valid token). A
// gathered row is computed in 64 bits and is absent (kOff: reads zero, its
// stores are dropped) unless the whole row lies inside the resource, so a
// row index far past the matrix can never wrap onto another row.
template <typename PT>
__device__ __forceinline__ uint32_t row_off(const PT& P, const TileInfo& t, const TileRows& tr, int n) {
  if (n >= t.cnt) return kOff;
  if (!tr.gather) return (uint32_t)((int64_t)n * tr.ld2);
  int row;
  if constexpr (PlanCap<PT>::self) {
    row = t.rows[n];
  } else if constexpr (PlanCap<PT>::rows) {
    typedef const int32_t __attribute__((address_space(4)))* KRow;
    const auto* kb = (const char __attribute__((address_space(4)))*)__builtin_amdgcn_kernarg_segment_ptr();
    row = reinterpret_cast<KRow>(kb + PlanCap<PT>::kOffRows)[t.p0 + n];
  } else {
    row = P.token_rows[t.p0 + n];
  }
  const int64_t off = (int64_t)row * tr.ld2;
  return (off < 0 || off > tr.lim) ? kOff : (uint32_t)off;
}

// ---------------------------------------------------------------------------
// Grouping a request-order batch by adapter on the device (a stable counting
// sort: adapters in id order, the tokens of an adapter in request order,
// tokens without an active adapter last in key N, which gets no tiles).
// ---------------------------------------------------------------------------
// Wave-level exclusive scan of the tokens per key, cnt[0..N] (LDS): each lane
// takes a block of consecutive keys and the blocks' sums are scanned with
// shuffles. visit(j, key, first sorted position, first tile, tokens) runs
// for each of the lane's kPer slots j (key = lane * kPer + j; slots past
// key N carry no tokens). Returns the tile count (all lanes).
// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by
// 1, 2, 4 and 8 lanes inside each row of 16 (a lane shifted in from outside
// its row reads 0), then the last lane of row 0 added to row 1 (and of row 2
// to row 3), then the last lane of row 1 to rows 2 and 3. Lane shuffles,
// which go through the LDS crossbar, made the in-launch planner's scan
// about 0.3 us longer per launch.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return v;
}

template <typename F>
__device__ __forceinline__ int scan_keys(const int* cnt, int N, F&& visit) {
  constexpr int kPer = (kMaxGraphAdapters + 1 + 63) / 64;
  const int lane = threadIdx.x & 63;
  int c[kPer], ls = 0, lt = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = lane * kPer + j;
    c[j] = i <= N ? cnt[i] : 0;
    ls += c[j];
    lt += i < N ? (c[j] + kTileM - 1) / kTileM : 0;
  }
  const int ss = wave_incl_scan(ls), st = wave_incl_scan(lt);
  int tok = ss - ls, tile = st - lt;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = lane * kPer + j;
    visit(j, i, tok, tile, c[j]);
    tok += c[j];
    tile += i < N ? (c[j] + kTileM - 1) / kTileM : 0;
  }
  return __builtin_amdgcn_readlane(st, 63);
}

// Lane 0's 64-bit value in SGPRs. readfirstlane returns a signed int: each
// half goes back through uint32_t, or a low word with bit 31 set would be
// sign-extended over the high word.
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// An adapter takes part if its rank is in [1, max_rank] and both weight
// addresses are set; ids outside [0, N) and inactive adapters map to key N.
__device__ __forceinline__ bool adapter_active(int rank, int max_rank, uint64_t wptr, uint64_t vptr) {
  return rank >= 1 && rank <= max_rank && wptr != 0 && vptr != 0;
}

// Planning inside the launch. Every workgroup reads the ids (at most
// kSelfPlanTokens, kThreads apart per thread) and the adapter tables
// (thread i: adapter i) and counts the tokens per key; wave 0 scans the
// counts, picks the workgroup's item (for the split layouts, re-laid out for
// the tiles the batch has) and finds the key and the place of the item's
// tile among the key's tokens; the key's tokens are then ranked in request
// order to collect the tile's rows in L.rows. Five barriers. The scratch
// lives in LDS buffer 0, which the item reuses afterwards.
constexpr int kSelfKPT = kSelfPlanTokens / kThreads;
constexpr int kSelfCW = 4 * kSelfKPT;  // (token block, wave) pairs
struct SelfLds {
  int* cnt;       // [N + 1] tokens per key
  int* cw;        // [kSelfCW] tokens of the tile's key in each (block of kThreads tokens, wave)
  int* rank;      // [N] the adapter tables, with rank 0 for inactive adapters
  float* scale;   // [N]
  uint64_t* wp;   // [N]
  uint64_t* vp;   // [N]
  int* pick;      // item tile, chunk, kind, blocks per chunk; tile's key, place in the key, count, position
};
__device__ __forceinline__ SelfLds self_lds(const Lds& L) {
  constexpr int K1 = kMaxGraphAdapters + 1;
  static_assert((K1 + kSelfCW + 6 * kMaxGraphAdapters + 8) * 4 <= LdsBytes<1>::b0, "plan scratch fits buffer 0");
  uint64_t* q = reinterpret_cast<uint64_t*>(L.b0);
  SelfLds S;
  S.wp = q;
  S.vp = q + kMaxGraphAdapters;
  int* p = reinterpret_cast<int*>(q + 2 * kMaxGraphAdapters);
  S.rank = p;
  S.scale = reinterpret_cast<float*>(p + kMaxGraphAdapters);
  S.cnt = p + 2 * kMaxGraphAdapters;
  S.cw = S.cnt + K1;
  S.pick = S.cw + kSelfCW;
  return S;
}

struct SelfItem {
  FwdItem it;  // g < 0: no item
  TileInfo t;
};

// The item and tile of workgroup b. item0: its item in the host's layout
// (laid out for the most tiles), kept where re-laying out would not change
// the column chunks. old_epoch: thread 0's read of the epoch as it added the
// workgroup's share (dep mode), kept for the launch id.
template <typename PT>
__device__ __forceinline__ SelfItem self_plan(const PT& P, const Lds& L, int b, FwdItem item0, uint64_t old_epoch) {
  static_assert(kMaxGraphAdapters <= kThreads, "one adapter per thread");
  constexpr int K1 = kMaxGraphAdapters + 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = P.self_N, T = P.self_T;
  const SelfLds S = self_lds(L);
  // the global reads, all issued together
  int rk = 0;
  float sc = 0.f;
  uint64_t wp = 0, vp = 0;
  if (tid < N) {
    rk = P.self_ranks[tid];
    sc = P.self_scales[tid];
    wp = P.self_A[tid];
    vp = P.self_B[tid];
  }
  int key[kSelfKPT];
#pragma unroll
  for (int j = 0; j < kSelfKPT; ++j) {
    const int t = j * kThreads + tid;
    key[j] = t < T ? P.self_ids[t] : -1;
  }
  for (int i = tid; i < K1; i += kThreads) S.cnt[i] = 0;
  if (tid < N) {
    S.rank[tid] = adapter_active(rk, P.self_max_rank, wp, vp) ? rk : 0;
    S.scale[tid] = sc;
    S.wp[tid] = wp;
    S.vp[tid] = vp;
  }
  if (tid == 0) *L.lid = (old_epoch >> kEpochShift) + 1;
  __syncthreads();
  // keys and the count per key
#pragma unroll
  for (int j = 0; j < kSelfKPT; ++j) {
    if (j * kThreads + tid < T) {
      const int id = key[j];
      key[j] = (id >= 0 && id < N && S.rank[id] > 0) ? id : N;
      atomicAdd(&S.cnt[key[j]], 1);
    }
  }
  __syncthreads();
  // wave 0: tile offsets per key, the item, and the key of the item's tile
  if (wave == 0) {
    constexpr int kPer = (kMaxGraphAdapters + 1 + 63) / 64;
    int kt[kPer], kk[kPer], kc[kPer];
    // (the tile count cannot exceed the bound the grid was laid out for;
    // the clamp keeps every item inside the workspace regardless)
    const int tiles = min(scan_keys(S.cnt, N, [&](int j, int i, int tok, int tile, int c) {
      kt[j] = tile;
      kk[j] = tok;
      kc[j] = i < N ? c : 0;  // key N (no adapter) has no tiles
    }), P.n_tiles);
    FwdItem it = item0;
    int nblk = P.nblk;
    if (self_relayout_needed(P.self_relayout, tiles, P.n_tiles)) {
      int nc;
      nblk = self_relayout(P.self_relayout, tiles, P.ks, (P.N + 31) >> 5, P.self_slots, P.grid, nc);
      it = fwd_item_at(P.mode, P.xcd_local, P.xcd_remap, P.grid, tiles, P.ks, nc, tiles * P.ks, tiles * nc, b);
    }
    if (it.g >= tiles) it.g = -1;  // a tile past the batch's
    if (lane == 0) {
      S.pick[0] = it.g;
      S.pick[1] = it.c;
      S.pick[2] = it.kind;
      S.pick[3] = nblk;
    }
    if (it.g >= 0) {
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int i = lane * kPer + q;
        if (i < N && it.g >= kt[q] && it.g < kt[q] + (kc[q] + kTileM - 1) / kTileM) {
          const int j0 = (it.g - kt[q]) * kTileM;
          S.pick[4] = i;
          S.pick[5] = j0;
          S.pick[6] = min(kTileM, kc[q] - j0);
          S.pick[7] = kk[q] + j0;
        }
      }
    }
  }
  __syncthreads();
  SelfItem R;
  R.it.g = __builtin_amdgcn_readfirstlane(S.pick[0]);
  R.it.c = __builtin_amdgcn_readfirstlane(S.pick[1]);
  R.it.kind = __builtin_amdgcn_readfirstlane(S.pick[2]);
  if (R.it.g < 0) return R;
  TileInfo& t = R.t;
  t.g = R.it.g;
  t.nblk = __builtin_amdgcn_readfirstlane(S.pick[3]);
  const int a = __builtin_amdgcn_readfirstlane(S.pick[4]);
  const int j0 = __builtin_amdgcn_readfirstlane(S.pick[5]);
  t.cnt = __builtin_amdgcn_readfirstlane(S.pick[6]);
  t.p0 = __builtin_amdgcn_readfirstlane(S.pick[7]);
  // this thread's tokens of key a, placed in request order: by lane within
  // a wave, then by wave, then by block of kThreads tokens
  int pre[kSelfKPT];
#pragma unroll
  for (int j = 0; j < kSelfKPT; ++j) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(key[j] == a);
    pre[j] = __builtin_popcountll(m & ((1ull << lane) - 1ull));
    if (lane == 0) S.cw[4 * j + wave] = __builtin_popcountll(m);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kSelfKPT; ++j) {
    if (key[j] == a) {
      int r = pre[j] - j0;
      for (int q = 0; q < 4 * j + wave; ++q) r += S.cw[q];
      if (r >= 0 && r < kTileM) L.rows[r] = j * kThreads + tid;
    }
  }
  t.adapter = a;
  t.rank = __builtin_amdgcn_readfirstlane(S.rank[a]);
  t.scale = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, S.scale[a])));
  t.wptr = uniform64(S.wp[a]);
  t.vptr = uniform64(S.vp[a]);
  t.slot = 0;
  t.proj = 0;
  t.rows = L.rows;
  t.lid = uniform64(*L.lid);
  __syncthreads();
  return R;
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
  bool xs;                      // x rows streamed (read by this item alone)
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
  if (C.xs) {
#pragma unroll
    for (int j = 0; j < G::NBX / 4; ++j)
      load_lds16_stream(C.xr, base + 4u * j * G::BS, kv ? C.roff[j] + kbytes : kOff);
  } else {
#pragma unroll
    for (int j = 0; j < G::NBX / 4; ++j) load_lds16(C.xr, base + 4u * j * G::BS, kv ? C.roff[j] + kbytes : kOff);
  }
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
    C.xr = mk_rsrc_words(P.X, kGatherSpan);
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
  // one item per tile (large batches, u kept on chip): each x row is read by
  // this workgroup alone, so it is streamed (packed-training forward, 65536
  // tokens: 306 -> 299 us). Launches that split a tile's shrink into parts
  // measured the same or slower with streamed x (8192-token prefill at rank
  // 64: 57 -> 61 us), so they keep plain loads.
  C.xs = P.mode == kModeFusedTile && P.nc == 1;
#pragma unroll
  for (int b = 0; b < RB; ++b) acc[b] = zero_acc16();
  const int nch = __builtin_amdgcn_readfirstlane((ke - kb + G::KC - 1) / G::KC);
  if (nch <= 0) return;
  // every wave's loads of a chunk must have landed before any wave reads it:
  // wait for this wave's loads of the chunk (its later chunk may stay in
  // flight), then barrier. Before a buffer is loaded again, every wave's
  // reads of it must be done: wait for LDS reads, then barrier.
  auto step = [&](uint8_t* buf, int cc) __attribute__((always_inline)) {
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
// The 8 values of a lane are read as two 16-byte vectors (the tile holds
// 32 * RB columns, so every read is inside it) and the columns past the
// rank are zeroed in registers.
template <int RB>
__device__ __forceinline__ void build_pfrags(const float* Pl, int rank, int lane, PFrags<RB>& F) {
  const int n = lane & 31, h = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 2 * RB; ++kb) {
    const int k0 = 16 * kb + 8 * h;
    const float4 a = *reinterpret_cast<const float4*>(Pl + n * kLdp + k0);
    const float4 b = *reinterpret_cast<const float4*>(Pl + n * kLdp + k0 + 4);
    float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (k0 + e >= rank) f[e] = 0.f;
    split8(f, F.hi[kb], F.lo[kb]);
  }
}

// Staged expand, for items of many blocks: the item's columns [c0, c1) in
// chunks of CW columns. A chunk's
// 32 y rows and its CW rows of V (one contiguous span of V) are staged
// through LDS; every wave computes whole 32-column blocks from LDS, with the
// rows of a block permuted by colmap so that a lane owns two runs of 8
// contiguous bf16 of one y row; the results go back into the LDS y tile,
// which is then stored row-contiguously (whole rows per store instruction,
// where the register-only expand stores 32 bytes of each row).
template <int RB>
struct StgRegs {
  u32x4 y[Geo<RB>::YV];
  u32x4 v[Geo<RB>::VV];
};

template <int RB>
struct StgCtx {
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
__device__ __forceinline__ void stg_load(const StgCtx<RB>& C, int cs, StgRegs<RB>& R) {
  using G = Geo<RB>;
  constexpr int YPR = G::CW / 8;
  const int col = cs + 8 * (threadIdx.x % YPR);
  const bool cv = col < C.c1;
  const uint32_t cbytes = 2u * (uint32_t)col;
#pragma unroll
  for (int j = 0; j < G::YV; ++j) R.y[j] = bld16_stream(C.yr, cv ? C.yoff[j] + cbytes : kOff);
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
__device__ __forceinline__ void stg_to_lds(const StgCtx<RB>& C, int cs, const StgRegs<RB>& R,
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
__device__ __forceinline__ void stg_mfma(const StgCtx<RB>& C, const PFrags<RB>& F, int cs, uint16_t* ys,
                                         const uint16_t* vs, int wave, int lane) {
  using G = Geo<RB>;
  constexpr int NB = G::CW / 32;  // 32-column blocks per chunk
  constexpr int BW = NB / 4;      // blocks per wave
  const int m = lane & 31, h = lane >> 5;
  // all LDS reads first, then the blocks' MFMA chains interleaved so that
  // their latencies overlap; blocks past the item's columns are computed
  // into LDS columns that are never stored
  u32x4 vf[BW][2 * RB], y0[BW], y1[BW];
#pragma unroll
  for (int b = 0; b < BW; ++b) {
    const int col0 = 32 * (wave + 4 * b);
    const uint16_t* vrow = vs + (col0 + colmap(m)) * G::RP + 8 * h;
#pragma unroll
    for (int kb = 0; kb < 2 * RB; ++kb)
      if (kb < C.kbn) vf[b][kb] = ld16(vrow + 16 * kb);
    // token m, columns col0 + 8h + [0, 8) and col0 + 16 + 8h + [0, 8)
    const uint16_t* yr = ys + m * G::CWP + col0 + 8 * h;
    y0[b] = ld16(yr);
    y1[b] = ld16(yr + 16);
  }
  f32x16 acc[BW];
#pragma unroll
  for (int b = 0; b < BW; ++b) acc[b] = zero_acc16();
#pragma unroll
  for (int kb = 0; kb < 2 * RB; ++kb)
    if (kb < C.kbn) {
#pragma unroll
      for (int b = 0; b < BW; ++b) acc[b] = mfma32(as_bf16x8(vf[b][kb]), F.hi[kb], acc[b]);
#pragma unroll
      for (int b = 0; b < BW; ++b) acc[b] = mfma32(as_bf16x8(vf[b][kb]), F.lo[kb], acc[b]);
    }
#pragma unroll
  for (int b = 0; b < BW; ++b) {
    uint16_t* yr = ys + m * G::CWP + 32 * (wave + 4 * b) + 8 * h;
    float f[8];
    unpack8(y0[b], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = f[i] + C.oscale * acc[b][i];
    st16(yr, pack8(f));
    unpack8(y1[b], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = f[i] + C.oscale * acc[b][8 + i];
    st16(yr + 16, pack8(f));
  }
  (void)cs;
}

template <int RB>
__device__ __forceinline__ void stg_store(const StgCtx<RB>& C, int cs, const uint16_t* ys) {
  using G = Geo<RB>;
  constexpr int YPR = G::CW / 8;
  constexpr int RPJ = kThreads / YPR;
  const int r0 = threadIdx.x / YPR, c = 8 * (threadIdx.x % YPR);
  const int col = cs + c;
  const bool cv = col < C.c1;
  const uint32_t cbytes = 2u * (uint32_t)col;
#pragma unroll
  for (int j = 0; j < G::YV; ++j)
    bst16_stream(C.yr, cv ? C.yoff[j] + cbytes : kOff, ld16(ys + (r0 + RPJ * j) * G::CWP + c));
}

template <int RB, typename PT>
__device__ __forceinline__ StgCtx<RB> stg_ctx(const PT& P, const TileInfo& t, int c) {
  using G = Geo<RB>;
  constexpr int YPR = G::CW / 8;
  constexpr int RPJ = kThreads / YPR;
  StgCtx<RB> C;
  const ProjView pv = proj_view(P, t.proj);
  const TileRows yt = tile_rows(pv.Y, pv.ldy, pv.N, P, t);
  C.yr = yt.r;
  const int r0 = threadIdx.x / YPR;
#pragma unroll
  for (int j = 0; j < G::YV; ++j) C.yoff[j] = row_off(P, t, yt, r0 + RPJ * j);
  C.ldv = ((t.rank + P.v_round - 1) / P.v_round) * P.v_round;
  C.vec16 = (C.ldv & 7) == 0;
  C.vr = mk_rsrc(v_ptr(P, t), (int64_t)pv.N * C.ldv * 2);
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
  expand_cols(pv.N, item_nblk(P, t), c, C.c0, C.c1);
  C.oscale = P.scale_in_shrink ? 1.f : t.scale;
  return C;
}

// Chunks of the expand whose loads are in flight (register sets).
template <int RB>
struct StgDepth {
  static constexpr int v = RB <= 2 ? 2 : 1;
};

// Runs the expand over the item's columns. R holds the loads of the first NE
// chunks, issued by the caller (so they can be issued before a wait).
template <int RB, int NE>
__device__ __forceinline__ void stg_run(const StgCtx<RB>& C, const PFrags<RB>& F, StgRegs<RB> (&R)[NE],
                                           uint8_t* stage) {
  using G = Geo<RB>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint16_t* ys = reinterpret_cast<uint16_t*>(stage);
  uint16_t* vs = ys + 32 * G::CWP;
  // a rank that ends half-way through a 16-wide k-step: the other half of
  // the last step is zero in every V row (written once; chunks never touch it)
  if (C.vec16 && (C.ldv & 8) && threadIdx.x < G::CW)
    st16(vs + threadIdx.x * G::RP + C.ldv, zero16());
  auto chunk = [&](int cs, StgRegs<RB>& Rq) __attribute__((always_inline)) {
    stg_to_lds<RB>(C, cs, Rq, ys, vs);
    lds_sync();
    stg_load<RB>(C, cs + NE * G::CW, Rq);  // past the range: reads nothing
    stg_mfma<RB>(C, F, cs, ys, vs, wave, lane);
    lds_sync();
    stg_store<RB>(C, cs, ys);
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

// Register-only expand, for items of at most one block per wave: the item's columns [c0, c1) in 32-column blocks, from registers.
// Wave w computes blocks w, w+4, ... of the item. Lane (m, h) loads the V row
// of output column col0 + colmap(m) (16 bytes per 16-wide k-step: k = 16 kb +
// 8 h .. +8), which is its A operand, and the two 16-byte runs of token m's
// y row that its 16 results update (columns col0 + 8 h and col0 + 16 + 8 h,
// 8 each), so the expand uses neither LDS nor barriers. The loads of the
// wave's next ExpDepth blocks are in flight while a block is computed.
template <int RB>
struct BlkRegs {
  u32x4 v[2 * RB];  // V rows (A fragments), one per 16-wide k-step
  u32x4 y[2];       // y runs of token m
};

// Blocks whose loads each wave keeps in flight (16, 24 and 40 VGPRs a block
// for RB = 1, 2, 4).
template <int RB>
struct ExpDepth {
  static constexpr int v = RB == 1 ? 4 : (RB == 2 ? 3 : 1);
};

template <int RB>
struct ExpCtx {
  __amdgpu_buffer_rsrc_t yr, vr;
  uint32_t yrow;  // byte offset of token m's y row, kOff past the tile
  int ldv;        // V row stride (elements)
  int rank, kbn;  // rank, k-steps of 16 that hold rank columns
  bool vec16;     // V rows are whole 16-byte vectors
  int c0, c1;     // column range of the item
  int nb;         // its 32-column blocks
  float oscale;
};

// Byte offset off, or one past every buffer (bit 31 set: the access reads
// zero or is dropped) when index >= limit. Plain arithmetic, so that no lane
// mask stays live across the expand loop.
__device__ __forceinline__ uint32_t off_if_below(uint32_t off, int index, int limit) {
  return off | ((uint32_t)((limit - 1 - index) >> 31) & 0x80000000u);
}

// Issues the loads of block j of the item (j >= nb: nothing is read).
template <int RB>
__device__ __forceinline__ void exp_load(const ExpCtx<RB>& C, int j, BlkRegs<RB>& R) {
  const int lane = threadIdx.x & 63, m = lane & 31, h = lane >> 5;
  const int col0 = C.c0 + 32 * j;
  const int vrow = col0 + colmap(m);
  // rows past the item (and so every row of a block past it) read zero
  const uint32_t vbase = off_if_below((uint32_t)(vrow * C.ldv * 2), vrow, C.c1);
#pragma unroll
  for (int kb = 0; kb < 2 * RB; ++kb) {
    if (kb >= C.kbn) continue;
    const int k0 = 16 * kb + 8 * h;
    if (C.vec16) {
      R.v[kb] = bld16(C.vr, off_if_below(vbase + 2u * (uint32_t)k0, k0, C.rank));
    } else {
      // rank not a multiple of 8 (V rows not 16-byte aligned): element
      // loads, zero past the rank. They are waited for here, so that this
      // rare layout holds no more registers in flight than the usual one.
      u32x4 v = zero16();
#pragma nounroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = bld2(C.vr, off_if_below(vbase + 2u * (uint32_t)(k0 + e), k0 + e, C.rank));
        const uint32_t sh = 16u * (uint32_t)(e & 1);
        if (e < 2) v[0] |= w << sh;
        else if (e < 4) v[1] |= w << sh;
        else if (e < 6) v[2] |= w << sh;
        else v[3] |= w << sh;
      }
      R.v[kb] = v;
    }
  }
  // y: token rows past the tile have yrow = kOff (bit 31 set) already
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int col = col0 + 16 * r + 8 * h;
    R.y[r] = bld16_stream(C.yr, off_if_below(C.yrow + 2u * (uint32_t)col, col, C.c1));
  }
}

// Computes block j from its loaded registers and stores its y runs.
template <int RB>
__device__ __forceinline__ void exp_block(const ExpCtx<RB>& C, const PFrags<RB>& F, int j,
                                          const BlkRegs<RB>& R) {
  const int lane = threadIdx.x & 63, h = lane >> 5;
  f32x16 acc = zero_acc16();
#pragma unroll
  for (int kb = 0; kb < 2 * RB; ++kb)
    if (kb < C.kbn) {
      acc = mfma32(as_bf16x8(R.v[kb]), F.hi[kb], acc);
      acc = mfma32(as_bf16x8(R.v[kb]), F.lo[kb], acc);
    }
  const int col0 = C.c0 + 32 * j;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int col = col0 + 16 * r + 8 * h;
    float f[8];
    unpack8(R.y[r], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = f[i] + C.oscale * acc[8 * r + i];
    bst16_stream(C.yr, off_if_below(C.yrow + 2u * (uint32_t)col, col, C.c1), pack8(f));
  }
}

template <int RB, typename PT>
__device__ __forceinline__ ExpCtx<RB> exp_ctx(const PT& P, const TileInfo& t, int c) {
  ExpCtx<RB> C;
  const ProjView pv = proj_view(P, t.proj);
  const TileRows yt = tile_rows(pv.Y, pv.ldy, pv.N, P, t);
  C.yr = yt.r;
  C.yrow = row_off(P, t, yt, threadIdx.x & 31);
  C.ldv = ((t.rank + P.v_round - 1) / P.v_round) * P.v_round;
  C.vec16 = (C.ldv & 7) == 0;
  C.vr = mk_rsrc(v_ptr(P, t), (int64_t)pv.N * C.ldv * 2);
  C.rank = t.rank;
  C.kbn = (t.rank + 15) >> 4;
  expand_cols(pv.N, item_nblk(P, t), c, C.c0, C.c1);
  C.nb = (C.c1 - C.c0 + 31) >> 5;
  C.oscale = P.scale_in_shrink ? 1.f : t.scale;
  return C;
}

// Issues the loads of the wave's first ExpDepth blocks.
template <int RB, int NE>
__device__ __forceinline__ void exp_prefetch(const ExpCtx<RB>& C, BlkRegs<RB> (&R)[NE]) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 0; d < NE; ++d) exp_load<RB>(C, wave + 4 * d, R[d]);
}

// Runs the wave's blocks. R holds the loads of its first NE blocks (issued by
// the caller, so that they can be in flight during a wait).
template <int RB, int NE>
__device__ __forceinline__ void expand_run(const ExpCtx<RB>& C, const PFrags<RB>& F, BlkRegs<RB> (&R)[NE]) {
  const int wave = threadIdx.x >> 6;
  for (int i = 0; wave + 4 * i < C.nb; i += NE) {
#pragma unroll
    for (int d = 0; d < NE; ++d) {
      const int j = wave + 4 * (i + d);
      if (j < C.nb) {
        exp_block<RB>(C, F, j, R[d]);
        exp_load<RB>(C, j + 4 * NE, R[d]);  // past the item: reads nothing
      }
    }
  }
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

// Items of at most one 32-column block per wave take the register-only
// expand (no LDS stage or barriers); longer ones the staged expand, whose
// stores cover whole rows.
template <int RB>
__device__ __forceinline__ bool direct_expand(int nblk) { return nblk <= 4; }

template <int RB, typename PT>
__device__ __forceinline__ void expand_from_lds(const PT& P, const TileInfo& t, int c, const float* Pl,
                                                uint8_t* stage) {
  PFrags<RB> F;
  if (direct_expand<RB>(item_nblk(P, t))) {
    const ExpCtx<RB> C = exp_ctx<RB>(P, t, c);
    constexpr int NE = ExpDepth<RB>::v;
    BlkRegs<RB> R[NE];
    exp_prefetch<RB, NE>(C, R);
    build_pfrags<RB>(Pl, t.rank, threadIdx.x & 63, F);
    expand_run<RB, NE>(C, F, R);
  } else {
    const StgCtx<RB> C = stg_ctx<RB>(P, t, c);
    constexpr int NE = StgDepth<RB>::v;
    StgRegs<RB> R[NE];
#pragma unroll
    for (int q = 0; q < NE; ++q) stg_load<RB>(C, C.c0 + q * Geo<RB>::CW, R[q]);  // empty ranges read nothing
    build_pfrags<RB>(Pl, t.rank, threadIdx.x & 63, F);
    stg_run<RB, NE>(C, F, R, stage);
  }
}

// kModeFusedTile: full shrink of one tile on chip, then its n-chunk c.
template <int RB, typename PT>
__device__ __forceinline__ void item_fused_tile(const PT& P, const Lds& L, const TileInfo& t, int c) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  f32x16 acc[RB];
  shrink_lds<RB>(P, t, 0, P.K, L, acc);
  const float ps = P.scale_in_shrink ? t.scale : 1.f;
  float* Pl = L.Pl();
  reduce_waves<RB>(L.red(), acc, wave, lane, [&](int k, int n, float v) __attribute__((always_inline)) { Pl[n * kLdp + k] = v * ps; });
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

// ---------------------------------------------------------------------------
// Hand-off of split-shrink parts (kModeFusedDep). A part is published by
// storing it, waiting until every store of the workgroup has been performed,
// and then storing its stamp (launch id << 8 | XCD of the writer). An expand
// waits until every part of its tile carries the current launch id, then
// reads the parts. Launch ids are unique, so a stamp left by an earlier call
// never matches, and no counter has to be returned to zero.
// Stamps and parts are stored and read with device scope (the reads miss
// both the CU's L1 and a stale L2 line), in every layout: in the XCD-local
// one too, where plain part stores and loads would meet in that XCD's L2,
// the device-scope loads measured faster (decode q, 2560 -> 2560: the part
// loads 1.7 -> 0.9 us, the launch 10.3 -> 9.4 us in a phase trace), and a
// part written on another XCD is then just as valid. Each stamp has a cache
// line to itself: with eight stamps to a line, the 30-40 expands of a tile
// polling them and the parts storing them met on one line (decode gate_up,
// 2560 -> 19456: 15.7 -> 14.7 us).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t xcc_id() {
  return (uint32_t)__builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11));  // HW_REG_XCC_ID[3:0]
}
constexpr int kAuxDev = 16;  // sc1: device scope

// The id that stamps this launch's parts: from the host; for batches planned
// inside the launch, the one the workgroup took when it advanced the epoch;
// for batches planned by the plan kernel, from the epoch it has just advanced.
template <typename PT>
__device__ __forceinline__ uint64_t launch_id(const PT& P, const TileInfo& t) {
  if constexpr (PlanCap<PT>::self) return t.lid;
  if (P.dev_epoch) return uniform64(*P.dev_epoch >> kEpochShift);
  return P.launch_id;
}

template <typename PT>
__device__ __forceinline__ float* partial_ptr(const PT& P, int g, int c) {
  return P.partials + ((int64_t)g * P.ks + c) * kTileM * P.rpad;
}

// Stamp of part (g, c) as seen by this workgroup's thread.
template <typename PT>
__device__ __forceinline__ uint64_t load_stamp(const PT& P, int idx) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const __amdgpu_buffer_rsrc_t r = mk_rsrc(P.stamps, (int64_t)kMaxPartials * kStampStride);
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, idx * kStampStride, 0, kAuxDev);
  return ((uint64_t)v[1] << 32) | v[0];
}

// Sums tile t's ks parts in order q = 0, 1, ... into Pl (scaled), with the
// loads of several parts in flight together; device_scope: the parts were
// written with device-scope stores (read past the CU's L1 and a stale L2).
template <int RB, typename PT>
__device__ __forceinline__ void sum_parts_to_lds(const PT& P, const TileInfo& t, float* Pl, bool device_scope) {
  const float ps = P.scale_in_shrink ? t.scale : 1.f;
  constexpr int RC = 32 * RB;                  // rank columns of the P tile
  constexpr int EPT = kTileM * RC / kThreads;  // elements per thread
  // the loads of PD parts (all of them for the usual k split) are in flight
  // together
  const __amdgpu_buffer_rsrc_t r = mk_rsrc(partial_ptr(P, t.g, 0), (int64_t)P.ks * kTileM * P.rpad * 4);
  const uint32_t part_bytes = (uint32_t)(kTileM * P.rpad * 4);
  // a part is stored rank-major, P^T [rpad][32 tokens]: element e of the
  // first RC rows is (rank e / 32, token e % 32) at float offset e. A thread
  // loads 16-byte vectors (elements 4v .. 4v + 3, one rank, four tokens),
  // so the loads are contiguous across the workgroup
  constexpr int VPT = EPT / 4;  // vectors per thread
  float s[EPT];
  uint32_t off[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) off[j] = (uint32_t)((threadIdx.x + kThreads * j) * 16);
#pragma unroll
  for (int j = 0; j < EPT; ++j) s[j] = 0.f;
  constexpr int PD = 8 / RB;
  for (int q0 = 0; q0 < P.ks; q0 += PD) {
    u32x4 v[PD][VPT];
#pragma unroll
    for (int d = 0; d < PD; ++d)
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const uint32_t o = q0 + d < P.ks ? (uint32_t)(q0 + d) * part_bytes + off[j] : kOff;
        v[d][j] = device_scope ? __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, kAuxDev)
                               : __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0);
      }
#pragma unroll
    for (int d = 0; d < PD; ++d)
#pragma unroll
      for (int j = 0; j < VPT; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q0 + d < P.ks) {
            // through a named value: a bit cast of the vector element
            // itself is compiled as a read of element 0
            const uint32_t w = v[d][j][q];
            const float f = __builtin_bit_cast(float, w);
            s[4 * j + q] = (q0 + d == 0) ? f : s[4 * j + q] + f;
          }
  }
#pragma unroll
  for (int j = 0; j < VPT; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * (threadIdx.x + kThreads * j) + q;
      const int k = e / kTileM, n = e - k * kTileM;
      Pl[n * kLdp + k] = s[4 * j + q] * ps;
    }
  lds_sync();
}

// kModeShrink / kModeFusedDep phase A: shrink over k-chunk c.
template <int RB, typename PT>
__device__ __forceinline__ void item_shrink(const PT& P, const Lds& L, const TileInfo& t, int c) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int kb, ke;
  shrink_range(P.K, P.kchunk, c, kb, ke);
  f32x16 acc[RB];
  shrink_lds<RB>(P, t, kb, ke, L, acc);
  float* red = L.red();
  const float ps = P.scale_in_shrink ? t.scale : 1.f;
  if (P.mode == kModeShrink && P.ks == 1) {
    // the lambda takes plain values, not the plan (a reference to the kernel
    // argument held in a closure can make the compiler copy the plan to scratch)
    float* const U = P.U + (int64_t)t.p0 * P.ldu;
    const int64_t ldu = P.ldu;
    const int cnt = t.cnt, rank = t.rank;
    reduce_waves<RB>(red, acc, wave, lane, [&](int k, int n, float v) __attribute__((always_inline)) {
      if (n < cnt && k < rank) U[(int64_t)n * ldu + k] = v * ps;
    });
    return;
  }
  float* part = partial_ptr(P, t.g, c);
  if (P.mode == kModeFusedDep) {
    reduce_waves<RB>(red, acc, wave, lane, [&](int k, int n, float v) __attribute__((always_inline)) {
      __hip_atomic_store(part + k * kTileM + n, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    });
    asm volatile("" ::: "memory");
    wait_vmcnt<0>();  // this thread's part stores have been performed
    __syncthreads();  // ... and every thread's
    if (threadIdx.x == 0) {
      const uint64_t stamp = (launch_id(P, t) << 8) | xcc_id();
      __hip_atomic_store(P.stamps + (t.g * P.ks + c) * (kStampStride / 8), stamp, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  // kModeShrink, ks > 1: each chunk stores its part with device-scope
  // stores, waits until they are performed, and counts itself in the tile's
  // arrival counter; the last arriving chunk sums all parts in order (the
  // same ordered sum as the fused hand-off, several parts' loads in flight),
  // writes u and returns the counter to 0
  reduce_waves<RB>(red, acc, wave, lane, [&](int k, int n, float v) __attribute__((always_inline)) {
    __hip_atomic_store(part + k * kTileM + n, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  });
  asm volatile("" ::: "memory");
  wait_vmcnt<0>();  // this thread's part stores have been performed
  int* ctr = P.counters + kCtrTiles + t.g;
  __syncthreads();  // ... and every thread's
  if (threadIdx.x == 0) *L.flag = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (*L.flag != P.ks - 1) return;
  float* Pl = L.Pl();
  sum_parts_to_lds<RB>(P, t, Pl, true);
  store_u_from_lds(P, t, Pl);
  if (threadIdx.x == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// kModeFusedDep phase B: wait for the tile's parts, sum them in order,
// expand n-chunk c. If the parts do not all arrive within spin_ticks (their
// workgroups not resident), the item computes the same parts itself in the
// same order, so the result is identical and no wait is unbounded.
// Waits for the stamps of tile t's parts; on success sums the parts in order
// q = 0, 1, ... into Pl (scaled) and returns true.
template <int RB, typename PT>
__device__ __forceinline__ bool wait_and_sum_parts(const PT& P, const Lds& L, const TileInfo& t, float* Pl) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave == 0) {
    // lane q < ks watches the stamp of part q
    const bool mine = lane < P.ks;
    const int idx = t.g * P.ks + (mine ? lane : 0);
    const uint64_t want = launch_id(P, t);
    const uint64_t t0 = wall_clock64();
    bool ready = false;
    while (true) {
      const uint64_t st = load_stamp(P, idx);
      const bool arrived = !mine || (st >> 8) == want;
      if (__builtin_amdgcn_ballot_w64(!arrived) == 0) {
        ready = true;
        break;
      }
      if (wall_clock64() - t0 > (uint64_t)P.spin_ticks) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) *L.flag = ready ? 1 : 0;
  }
  __syncthreads();
  if (!*L.flag) return false;
  sum_parts_to_lds<RB>(P, t, Pl, true);
  return true;
}


template <int RB, typename PT>
__device__ __forceinline__ void item_expand_wait(const PT& P, const Lds& L, const TileInfo& t, int c) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* Pl = L.Pl();
  // y rows and expand weights do not depend on the shrink: the first loads
  // are issued before waiting
  bool done = false;
  if (direct_expand<RB>(item_nblk(P, t))) {
    const ExpCtx<RB> C = exp_ctx<RB>(P, t, c);
    constexpr int NE = ExpDepth<RB>::v;
    BlkRegs<RB> R[NE];
    exp_prefetch<RB, NE>(C, R);
    if (wait_and_sum_parts<RB>(P, L, t, Pl)) {
      if (P.write_u && c == 0) store_u_from_lds(P, t, Pl);
      PFrags<RB> F;
      build_pfrags<RB>(Pl, t.rank, lane, F);
      expand_run<RB, NE>(C, F, R);
      done = true;
    }
  } else {
    const StgCtx<RB> C = stg_ctx<RB>(P, t, c);
    constexpr int NE = StgDepth<RB>::v;
    StgRegs<RB> R[NE];
#pragma unroll
    for (int q = 0; q < NE; ++q) stg_load<RB>(C, C.c0 + q * Geo<RB>::CW, R[q]);  // empty ranges read nothing
    if (wait_and_sum_parts<RB>(P, L, t, Pl)) {
      if (P.write_u && c == 0) store_u_from_lds(P, t, Pl);
      PFrags<RB> F;
      build_pfrags<RB>(Pl, t.rank, lane, F);
      stg_run<RB, NE>(C, F, R, L.b0);
      done = true;
    }
  }
  if (done) return;
  // Fallback. The early loads are dropped and issued again after the shrink
  // (a separate expand, so that they are not held in registers through it).
  // The chunk sums run in registers (each thread always receives the same
  // elements from the reduction) because the shrink reuses P's LDS buffer;
  // the last chunk's pass writes P.
  const float ps = P.scale_in_shrink ? t.scale : 1.f;
  float run[4 * RB];
  for (int q = 0; q < P.ks; ++q) {
    int kb, ke;
    shrink_range(P.K, P.kchunk, q, kb, ke);
    f32x16 acc[RB];
    shrink_lds<RB>(P, t, kb, ke, L, acc);
    int idx = 0;
    const bool last = q == P.ks - 1;
    reduce_waves<RB>(L.red(), acc, wave, lane, [&](int k, int n, float v) __attribute__((always_inline)) {
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
    case kItemShrink: item_shrink<RB>(P, L, t, c); break;
    case kItemExpand: item_expand<RB>(P, L, t, c); break;
    case kItemFusedTile: item_fused_tile<RB>(P, L, t, c); break;
    default: item_expand_wait<RB>(P, L, t, c); break;
  }
}

template <int RBMAX, typename PT>
__global__ __launch_bounds__(kThreads, 2) void sgmv_fwd_kernel(PT P) {
  __shared__ alignas(16) uint8_t lds_b0[LdsBytes<RBMAX>::b0];
  __shared__ alignas(16) uint8_t lds_b1[LdsBytes<RBMAX>::b1];
  __shared__ TileInfo lds_ti;
  __shared__ int lds_flag;
  __shared__ int lds_rows[kTileM];
  __shared__ uint64_t lds_lid;
  const Lds L{lds_b0, lds_b1, &lds_ti, &lds_flag, lds_rows, &lds_lid};
  const int b = blockIdx.x;
  // Word 16 i of the plan (the kernel's argument): naming one word of each
  // 64-byte line in a batch of scalar loads brings that line into the scalar
  // cache, so that later, dependent reads of it do not go to memory.
  typedef const uint32_t __attribute__((address_space(4)))* KWord;
  const auto* kb = (const char __attribute__((address_space(4)))*)__builtin_amdgcn_kernarg_segment_ptr();
  const auto line = [&](int i) __attribute__((always_inline)) {
    return 64 * i < (int)sizeof(PT) ? *reinterpret_cast<KWord>(kb + 64 * i) : 0u;
  };
  if constexpr (PlanCap<PT>::self) {
    // the header lines that planning inside the launch and the items read
    // (the addresses of the ids, tables and epoch, the layout), in one batch
    // before the epoch is advanced
    static_assert(__builtin_offsetof(FwdPlanSelf, self_slots) < 5 * 64, "the planner's fields in lines 0-4");
    asm volatile("" ::"s"(line(0)), "s"(line(1)), "s"(line(2)), "s"(line(3)), "s"(line(4)), "s"(P.mode),
                 "s"(P.grid), "s"(P.dev_epoch));
  }
  // A launch planned inside itself with the split hand-off advances the
  // epoch by kEpochCall in all: every workgroup, with or without an item,
  // adds its share once (workgroup 0 the rest); the value read back gives
  // every workgroup the same launch id.
  static_assert(kEpochSlots <= 64, "workgroup 0's first wave covers the slots");
  uint64_t old_epoch = 0;
  if (PlanCap<PT>::self && P.mode == kModeFusedDep) {
    constexpr int kSlotWords = kEpochStride / 8;
    if (threadIdx.x == 0) {
      const int s = b % kEpochSlots;
      const uint64_t n_s = (uint64_t)((P.grid - 1 - s) / kEpochSlots + 1);  // workgroups of slot s
      old_epoch = __hip_atomic_fetch_add(P.dev_epoch + s * kSlotWords, b == s ? kEpochCall - (n_s - 1) : 1ull,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (b == 0 && (int)threadIdx.x >= P.grid && threadIdx.x < kEpochSlots) {
      // slots no workgroup uses (grids under kEpochSlots) advance in full
      __hip_atomic_fetch_add(P.dev_epoch + threadIdx.x * kSlotWords, kEpochCall, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // Read the launch parameters that select the item and its tile in one
  // batch of scalar loads: left to itself the compiler loads them one branch
  // at a time, a memory round trip each, before the item's first data load.
  // A small plan found on the host (at most 17 lines of 64 bytes) is also
  // read one word per line in that batch, so that the later, dependent reads
  // of the tile lookup and of the items (a segment's entries, its weight
  // addresses, the matrices' addresses) hit the scalar cache instead of
  // going to memory one after the other (decode gate_up, 2560 -> 19456:
  // 14.8 -> 13.9 us; q and o unchanged).
  if constexpr (!PlanCap<PT>::self && PlanCap<PT>::v <= kSmallSeg) {
    static_assert(sizeof(FwdPlanT<kSmallSeg>) <= 17 * 64, "one word per line of the plan");
    asm volatile("" ::"s"(line(0)), "s"(line(1)), "s"(line(2)), "s"(line(3)), "s"(line(4)), "s"(line(5)),
                 "s"(line(6)), "s"(line(7)), "s"(line(8)), "s"(line(9)), "s"(line(10)), "s"(line(11)),
                 "s"(line(12)), "s"(line(13)), "s"(line(14)), "s"(line(15)), "s"(line(16)), "s"(P.mode),
                 "s"(P.xcd_local), "s"(P.xcd_remap), "s"(P.n_tiles), "s"(P.ks), "s"(P.nc), "s"(P.n_items_a),
                 "s"(P.n_items_b), "s"(P.grid), "s"(P.n_seg), "s"(P.ptrs_in_plan), "s"(P.seg_tile0[0]),
                 "s"(P.seg_tok0[0]), "s"(P.seg_ntok[0]));
  } else {
    asm volatile("" ::"s"(P.mode), "s"(P.xcd_local), "s"(P.xcd_remap), "s"(P.n_tiles), "s"(P.ks),
                 "s"(P.nc), "s"(P.n_items_a), "s"(P.n_items_b), "s"(P.grid), "s"(P.n_seg),
                 "s"(P.ptrs_in_plan), "s"(P.seg_tile0[0]), "s"(P.seg_tok0[0]), "s"(P.seg_ntok[0]));
  }
  if constexpr (PlanCap<PT>::self) {
    // every workgroup plans: its item depends on the tiles the batch has
    const SelfItem R = self_plan(P, L, b, fwd_item(P, b), old_epoch);
    if (R.it.g < 0) return;  // no item, or a tile past the batch's
    const TileInfo& t = R.t;
    if (RBMAX == 1 || t.rank <= 32) run_item<1>(P, L, t, R.it.kind, R.it.c);
    else if (RBMAX == 2 || t.rank <= 64) run_item<(RBMAX >= 2 ? 2 : 1)>(P, L, t, R.it.kind, R.it.c);
    else run_item<RBMAX>(P, L, t, R.it.kind, R.it.c);
  } else {
    const FwdItem it = fwd_item(P, b);
    const int g = it.g, c = it.c, kind = it.kind;
    if (g >= 0) {
      const TileInfo t = tile_info(P, g, L.ti);
      if (t.cnt <= 0) return;  // a tile past the count of a batch planned on the device
      if (RBMAX == 1 || t.rank <= 32) run_item<1>(P, L, t, kind, c);
      else if (RBMAX == 2 || t.rank <= 64) run_item<(RBMAX >= 2 ? 2 : 1)>(P, L, t, kind, c);
      else run_item<RBMAX>(P, L, t, kind, c);
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
// wptr / vptr (or null): per segment weight addresses for small plans whose
// header sets ptrs_in_plan.
// Copies the segment table of a small launch (and its weight addresses, or
// zeros) from the host plan.
static void fill_small_plan(FwdPlanT<kSmallSeg>& Q, const FwdPlan& P, const uint64_t* wptr,
                            const uint64_t* vptr) {
  static_cast<FwdHeader&>(Q) = static_cast<const FwdHeader&>(P);
  for (int i = 0; i < P.n_seg; ++i) {
    Q.seg_wptr[i] = wptr ? wptr[i] : 0;
    Q.seg_vptr[i] = vptr ? vptr[i] : 0;
    Q.seg_tok0[i] = P.seg_tok0[i];
    Q.seg_ntok[i] = P.seg_ntok[i];
    Q.seg_tile0[i] = P.seg_tile0[i];
    Q.seg_adapter[i] = P.seg_adapter[i];
    Q.seg_scale[i] = P.seg_scale[i];
    Q.seg_rank[i] = P.seg_rank[i];
    Q.seg_slot[i] = P.seg_slot[i];
    Q.seg_proj[i] = P.seg_proj[i];
  }
}

hipError_t launch_fwd(const FwdPlan& P, int rbmax, hipStream_t stream, const uint64_t* wptr,
                      const uint64_t* vptr, const int32_t* rows, int n_rows) {
  if (P.self_ids) {
    FwdPlanSelf Q{};
    static_cast<FwdHeader&>(Q) = static_cast<const FwdHeader&>(P);
    return launch_fwd_t(Q, rbmax, stream);
  }
  if (rows) {
    // the caller guarantees n_seg <= kSmallSeg and n_rows <= kPlanRows
    FwdPlanRows Q{};
    fill_small_plan(Q, P, wptr, vptr);
    for (int i = 0; i < n_rows; ++i) Q.rows[i] = rows[i];
    return launch_fwd_t(Q, rbmax, stream);
  }
  if (P.n_seg <= kSmallSeg) {
    FwdPlanT<kSmallSeg> Q{};
    fill_small_plan(Q, P, wptr, vptr);
    return launch_fwd_t(Q, rbmax, stream);
  }
  return launch_fwd_t(P, rbmax, stream);
}

}  // namespace lora

namespace lora {

// ---------------------------------------------------------------------------
// Device-side planning (one workgroup): groups a request-order batch into
// per-adapter segments with a stable counting sort (adapters in id order,
// the tokens of an adapter in request order, tokens without an active adapter
// last), cuts the segments into 32-token tiles and advances the workspace
// epoch that stamps the following launch's hand-off by kEpochCall. Ids
// outside [0, N) and tokens of inactive adapters are left out of every tile.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPlanThreads) void dev_plan_kernel(DevPlanArgs a) {
  __shared__ int cnt[kMaxGraphAdapters + 1];
  __shared__ int start[kMaxGraphAdapters + 1];
  __shared__ int tile0[kMaxGraphAdapters + 1];
  __shared__ int wave_cnt[kPlanThreads / 64][kMaxGraphAdapters + 1];
  __shared__ int act[kMaxGraphAdapters];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.N;
  // every global read is issued before the first barrier: the epoch's slots
  // (one per thread), one adapter's table entries per thread (N <= 256 <
  // kPlanThreads) and the first chunk's ids, which stay in registers for
  // both passes
  uint64_t* const slot = a.epoch + (tid % kEpochSlots) * (kEpochStride / 8);
  const uint64_t epoch0 = tid < kEpochSlots ? *slot : 0;
  int rk = 0;
  float sc = 0.f;
  uint64_t wp = 0, vp = 0;
  if (tid < N) {
    rk = a.ranks[tid];
    sc = a.scales[tid];
    wp = a.A_ptrs[tid];
    vp = a.B_ptrs[tid];
  }
  const int id0 = tid < a.T ? a.ids[tid] : -1;
  for (int i = tid; i <= N; i += kPlanThreads) cnt[i] = 0;
  if (tid < N) act[tid] = adapter_active(rk, a.max_rank, wp, vp) ? 1 : 0;
  __syncthreads();
  auto key_of_id = [&](int id) { return (id >= 0 && id < N && act[id]) ? id : N; };
  // pass 1: tokens per key
  for (int t = tid; t < a.T; t += kPlanThreads) atomicAdd(&cnt[key_of_id(t == tid ? id0 : a.ids[t])], 1);
  __syncthreads();
  // token and tile offsets per key
  if (wave == 0) {
    const int tiles = scan_keys(cnt, N, [&](int, int i, int tok, int tile, int) {
      if (i <= N) {
        start[i] = tok;
        tile0[i] = tile;
      }
    });
    if (lane == 0) *a.count = min(tiles, a.max_tiles);
  }
  if (tid < kEpochSlots) *slot = epoch0 + kEpochCall;
  __syncthreads();
  // tiles: thread i writes adapter i's, from the table entries it holds
  if (tid < N) {
    const int c = cnt[tid];
    for (int j = 0; j < c; j += kTileM) {
      const int g = tile0[tid] + j / kTileM;
      if (g >= a.max_tiles) break;
      DevTile d;
      d.tok0 = start[tid] + j;
      d.cnt = min(kTileM, c - j);
      d.adapter = tid;
      d.rank = rk;
      d.scale = sc;
      d.pad = 0;
      d.wptr = wp;
      d.vptr = vp;
      a.tiles[g] = d;
    }
  }
  // pass 2: stable positions, a chunk of kPlanThreads tokens at a time. Within
  // a wave, the lanes of one key are ranked by lane order; the waves of a
  // chunk follow in order; earlier chunks come first.
  for (int c0 = 0; c0 < a.T; c0 += kPlanThreads) {
    for (int i = lane; i <= N; i += 64) wave_cnt[wave][i] = 0;
    const int t = c0 + tid;
    const int key = t < a.T ? key_of_id(c0 == 0 ? id0 : a.ids[t]) : -1;
    int rank_in_wave = 0;
    uint64_t todo = __builtin_amdgcn_ballot_w64(key >= 0);
    while (todo) {
      const int leader = __builtin_ctzll(todo);
      const int k = __builtin_amdgcn_readlane(key, leader);
      const uint64_t m = __builtin_amdgcn_ballot_w64(key == k);
      if (key == k) rank_in_wave = __builtin_popcountll(m & ((1ull << lane) - 1ull));
      if (lane == leader) wave_cnt[wave][k] = __builtin_popcountll(m);
      todo &= ~m;
    }
    __syncthreads();
    // per key: the waves' offsets in order (one thread per key)
    for (int k = tid; k <= N; k += kPlanThreads) {
      int s = start[k];
      for (int w = 0; w < kPlanThreads / 64; ++w) {
        const int n = wave_cnt[w][k];
        wave_cnt[w][k] = s;
        s += n;
      }
      start[k] = s;
    }
    __syncthreads();
    if (key >= 0) {
      const int pos = wave_cnt[wave][key] + rank_in_wave;
      if (pos >= 0 && pos < a.T) a.perm[pos] = t;  // always inside; the check keeps it so
    }
    __syncthreads();
  }
}

hipError_t launch_dev_plan(const DevPlanArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(dev_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lora
