// lora_plan.h -- launch plans shared by the host planner and the gfx950
// kernels of the multi-adapter LoRA library. Internal; not part of the ABI.
//
// A plan travels by value as the kernel argument, so a call needs no
// host-to-device copy of metadata: segment tables live in the kernel-argument
// segment and are read with scalar loads.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

constexpr int kThreads = 256;  // 4 wave64 per workgroup
constexpr int kTileM = 32;     // tokens per tile (the N side of a 32x32 MFMA)
constexpr int kMaxSeg = 128;   // segments per forward launch
constexpr int kMaxJobs = 64;   // adapter jobs per weight-gradient launch
constexpr int kMaxJobSeg = 128;
constexpr int kMaxPartials = 2048;  // (tile, k-chunk) parts in split modes (bounds the workspace)
constexpr int kMaxProj = 4;         // projections over one x in one fused launch
// Span (bytes) of the buffer resource over a whole matrix whose rows are
// gathered through a token-row table: a row whose bytes would end past it is
// treated as absent by the kernels, and the host rejects batches whose T
// rows cannot fit in it.
constexpr int64_t kGatherSpan = 0x7ffffff0;

// Forward-style launch modes (also used for the backward du/dx pass).
enum FwdMode : int32_t {
  kModeShrink = 0,     // items: (tile, k-chunk). ks == 1 writes U; ks > 1: last arriver sums
  kModeExpand = 1,     // items: (tile, n-chunk). U is read from memory
  kModeFusedTile = 2,  // items: (tile, n-chunk). Each computes the tile's full shrink on chip
  kModeFusedDep = 3,   // items [0, a): (tile, k-chunk) shrink parts; [a, a+b): (tile, n-chunk)
                       // expands that wait for the parts' stamps, then sum the parts
};

// Counter layout inside the workspace (int32 words): per-tile arrival
// counters of split shrink-only calls. The part stamps of kModeFusedDep
// follow at byte offset kStampOffset: one uint64 per (tile, k-chunk), each
// on a cache line of its own (kStampStride bytes apart), so that the
// expands polling one part's stamp do not share a line with the polls and
// stores of other parts' stamps.
constexpr int kCtrTiles = 64;        // per-tile arrival counters start here
constexpr int kStampOffset = 4096;   // bytes from the counters to the stamps
constexpr int kStampStride = 128;    // bytes from one part's stamp to the next
// The epoch of device-planned calls: kEpochSlots uint64 words, one per
// kEpochStride bytes. Every call adds 1 << kEpochShift to every slot, so
// between calls all slots hold the same multiple of it, whose high bits
// count the calls (the id of the n-th call is n, never 0). A call planned
// inside its launch spreads each slot's sum over the workgroups that use
// the slot (workgroup b uses slot b % kEpochSlots; each adds 1, the first of
// a slot the rest), so any value a workgroup reads while adding its share
// shifts down to the same count, and the adds of a launch are spread over
// kEpochSlots addresses instead of piling up on one.
constexpr int kEpochShift = 20;
constexpr uint64_t kEpochCall = 1ull << kEpochShift;
constexpr int kEpochSlots = 64;
constexpr int kEpochStride = 128;  // bytes between slots (one cache line each)
// Device-planned calls of at most this many tokens are planned inside the
// fused launch (4 ids per thread of a workgroup), larger ones by the plan kernel.
constexpr int kSelfPlanTokens = 1024;

// One 32-token tile of a batch planned on the device (lora_sgmv_fused_graph):
// written by the plan kernel into the workspace, read by the fused kernel.
struct DevTile {
  int32_t tok0;     // first sorted position
  int32_t cnt;      // tokens (1..32)
  int32_t adapter;
  int32_t rank;
  float scale;
  int32_t pad;
  uint64_t wptr;    // shrink weight A_i
  uint64_t vptr;    // expand weight B_i
};

struct FwdHeader {
  const uint16_t* X;  // shrink input rows, bf16 (x forward, dy backward)
  int64_t ldx;
  uint16_t* Y;  // expand in/out rows, bf16 (y forward, dx backward)
  int64_t ldy;
  float* U;  // fp32 [T, ldu] sorted positions: input (expand) / output (shrink, save)
  int64_t ldu;
  const uint64_t* Wtab;  // per adapter: shrink weight [rank, K] row-major (ld = K); or null
  const uint64_t* Vtab;  // per adapter: expand weight [N, ldv] row-major; or null
  const uint16_t* Wslots;  // used when Wtab is null: slot s at Wslots + s * w_slot_elems
  const uint16_t* Vslots;
  int64_t w_slot_elems;
  int64_t v_slot_elems;
  const int32_t* token_rows;  // row of X/Y for each sorted position, or null
  float* partials;            // split-K partial sums [tile][ks][rpad][32] (rank-major)
  int32_t* counters;          // shrink-only arrival counters (zero on entry and on exit)
  uint64_t* stamps;           // kModeFusedDep: stamp of each shrink part ((launch_id << 8) | XCD)
  uint64_t launch_id;         // unique per launch (56 bits, never 0)
  int32_t K;                  // shrink reduction length
  int32_t N;                  // expand output width
  int32_t v_round;            // expand weight row stride = round_up(rank, v_round)
  int32_t mode;
  int32_t scale_in_shrink;  // 1: u = s * (W x) and expand unscaled; 0: y += s * V u
  int32_t write_u;          // kModeFusedTile/kModeFusedDep: also store U
  int32_t n_seg;
  int32_t n_tiles;
  int32_t ks;        // k-chunks per tile
  int32_t kchunk;    // elements per k-chunk (multiple of 8)
  int32_t nc;        // n-chunks per tile
  int32_t nblk;      // 32-column blocks per n-chunk
  int32_t rpad;      // row length of a partial tile (multiple of 32)
  int32_t n_items_a;
  int32_t n_items_b;
  int32_t xcd_remap;    // 1: map consecutive items of phase A to the same XCD
  int32_t xcd_local;    // kModeFusedDep: all items of a tile run on XCD (tile % 8)
  int32_t grid;         // launched workgroups
  int32_t spin_ticks;   // wall-clock ticks an expand waits before computing the shrink itself
  int32_t ptrs_in_plan; // small plans: weight addresses are in seg_wptr / seg_vptr
  // Batches planned on the device: the tiles, their count and the launch id
  // come from the workspace (written by the plan kernel just before), and
  // n_tiles above is only the bound the grid was laid out for. Null otherwise.
  const DevTile* dev_tiles;
  const int32_t* dev_count;
  // The workspace epoch of device-planned calls (both kinds below): slot 0
  // of kEpochSlots; bits [kEpochShift, 64) count the calls on the workspace.
  uint64_t* dev_epoch;
  // Batches planned inside the launch (device-planned calls of at most
  // kSelfPlanTokens tokens): every workgroup groups the request-order ids
  // itself against the device adapter tables and keeps its own tile; the
  // split hand-off's launch id comes from the epoch, which every workgroup
  // advances. Null otherwise.
  const int32_t* self_ids;
  const uint64_t* self_A;
  const uint64_t* self_B;
  const int32_t* self_ranks;
  const float* self_scales;
  int32_t self_T;
  int32_t self_N;
  int32_t self_max_rank;
  // How such a launch re-lays its split layout out for the tiles the batch
  // turns out to have (the grid, laid out for the most tiles, and the k
  // split stay): 0 keeps the host layout, 1 the XCD-local and 2 the spread
  // small-batch layouts with the column chunks per tile recomputed
  // (self_relayout); self_slots = resident workgroups of the GPU.
  int32_t self_relayout;
  int32_t self_slots;
  // Projections 1 .. kMaxProj-1 of a multi-projection launch (several
  // LoRA-wrapped projections over the same x); projection 0 uses Y, ldy, N,
  // nblk, Wtab and Vtab above, and entry 0 of these arrays is unused.
  uint16_t* proj_Y[kMaxProj];
  int64_t proj_ldy[kMaxProj];
  const uint64_t* proj_Wtab[kMaxProj];
  const uint64_t* proj_Vtab[kMaxProj];
  int32_t proj_N[kMaxProj];
  int32_t proj_nblk[kMaxProj];
};

constexpr int kSmallSeg = 16;  // capacity of the small plan (decode batches)
constexpr int kPlanRows = 256; // token rows a small plan can carry (host copy of token_rows)

// Segment table of a launch (struct of arrays), CAP entries. Small plans can
// also carry each segment's weight addresses (taken from the caller's host
// copies of the pointer tables).
template <int CAP>
struct FwdPlanT : FwdHeader {
  static constexpr int kPtrCap = CAP <= kSmallSeg ? CAP : 1;
  uint64_t seg_wptr[kPtrCap];
  uint64_t seg_vptr[kPtrCap];
  int32_t seg_tok0[CAP];
  int32_t seg_ntok[CAP];
  int32_t seg_tile0[CAP];
  int32_t seg_adapter[CAP];
  float seg_scale[CAP];
  uint8_t seg_rank[CAP];
  uint8_t seg_slot[CAP];
  uint8_t seg_proj[CAP];  // projection of the segment (0 unless multi-projection)
};
using FwdPlan = FwdPlanT<kMaxSeg>;

// ---------------------------------------------------------------------------
// Item geometry of a forward-style launch, shared by the kernel (which runs
// it) and the host planner's inspection entry (which lists it for tests).
// ---------------------------------------------------------------------------
enum ItemKind : int32_t {
  kItemShrink = 0,      // shrink over k-chunk c of tile g
  kItemExpand = 1,      // expand column chunk c of tile g, U from memory
  kItemFusedTile = 2,   // tile g's whole shrink on chip, then column chunk c
  kItemExpandWait = 3,  // column chunk c of tile g after its shrink parts
};
struct FwdItem {
  int g;     // tile (-1: the workgroup has nothing to do)
  int c;     // k-chunk (shrink) or column chunk (expand kinds)
  int kind;  // ItemKind
};

// Item of workgroup b in a layout of n_tiles tiles, ks shrink parts and nc
// column chunks per tile (split modes: n_items_a parts, n_items_b expands).
__host__ __device__ __forceinline__ FwdItem fwd_item_at(int mode, int xcd_local, int xcd_remap, int grid,
                                                         int n_tiles, int ks, int nc, int n_items_a,
                                                         int n_items_b, int b) {
  FwdItem it{-1, 0, kItemShrink};
  if (mode == kModeFusedDep) {
    if (xcd_local) {
      // XCD x = b % 8 runs tiles x, x + 8, ...: their shrink parts first,
      // then their expands (workgroup b runs on XCD b % 8)
      const int x = b & 7, j = b >> 3;
      const int tx = (n_tiles - x + 7) >> 3;
      if (j < tx * ks) {
        const int i = j / ks;
        it = FwdItem{x + 8 * i, j - i * ks, kItemShrink};
      } else if (j < tx * (ks + nc)) {
        const int j2 = j - tx * ks, i = j2 / nc;
        it = FwdItem{x + 8 * i, j2 - i * nc, kItemExpandWait};
      }
    } else if (b < n_items_a) {
      const int g = b / ks;
      it = FwdItem{g, b - g * ks, kItemShrink};
    } else if (b < n_items_a + n_items_b) {
      const int i = b - n_items_a, g = i / nc;
      it = FwdItem{g, i - g * nc, kItemExpandWait};
    }
    return it;
  }
  int i = b;
  if (xcd_remap) {
    const int q = grid >> 3;
    i = (b & 7) * q + (b >> 3);
  }
  const int per = mode == kModeShrink ? ks : nc;
  const int kind = mode == kModeShrink ? kItemShrink : (mode == kModeExpand ? kItemExpand : kItemFusedTile);
  if (i < n_items_a) {
    const int g = i / per;
    it = FwdItem{g, i - g * per, kind};
  }
  return it;
}

// Item of workgroup b.
__host__ __device__ __forceinline__ FwdItem fwd_item(const FwdHeader& P, int b) {
  return fwd_item_at(P.mode, P.xcd_local, P.xcd_remap, P.grid, P.n_tiles, P.ks, P.nc, P.n_items_a, P.n_items_b,
                     b);
}

// Whether a launch planned inside itself re-lays out for `tiles` tiles (its
// grid laid out for max_tiles): the column chunks change with the tile count
// only through the tiles per XCD (kind 1, XCD-local) or the tiles (kind 2);
// otherwise the host's layout, whose items of tiles past the count are
// idle, is kept.
__host__ __device__ inline bool self_relayout_needed(int kind, int tiles, int max_tiles) {
  if (kind == 0 || tiles <= 0) return false;
  return kind == 1 ? ((tiles + 7) >> 3) != ((max_tiles + 7) >> 3) : tiles != max_tiles;
}

// Column chunks per tile of a launch planned inside itself, for the `tiles`
// tiles its batch has (1 <= tiles <= the tiles its grid was laid out for):
// the host's small-batch rule (about two resident workgroups per CU; for
// the XCD-local layout per XCD) on the actual tiles, clamped so that every
// item still falls inside the grid. kind: 1 XCD-local, 2 spread. Returns
// nblk (32-column blocks per chunk); nc = the chunks.
__host__ __device__ inline int self_relayout(int kind, int tiles, int ks, int nblocks, int slots, int grid,
                                             int& nc) {
  int n;
  if (kind == 1) {
    const int per_xcd = (tiles + 7) / 8;
    n = slots / 8 / per_xcd - ks;
    const int fit = grid / (8 * per_xcd) - ks;
    n = n < fit ? n : fit;
  } else {
    n = slots / tiles - ks;
    const int fit = grid / tiles - ks;
    n = n < fit ? n : fit;
  }
  n = n < nblocks ? n : nblocks;
  n = n > 1 ? n : 1;
  const int nblk = (nblocks + n - 1) / n;
  nc = (nblocks + nblk - 1) / nblk;
  return nblk;
}

// k range [kb, ke) of shrink part c.
__host__ __device__ __forceinline__ void shrink_range(int K, int kchunk, int c, int& kb, int& ke) {
  kb = c * kchunk;
  ke = K < kb + kchunk ? K : kb + kchunk;
}

// Column range [c0, c1) of expand chunk c of an output n columns wide that
// is cut into chunks of nblk 32-column blocks.
__host__ __device__ __forceinline__ void expand_cols(int n, int nblk, int c, int& c0, int& c1) {
  const int nblocks = (n + 31) >> 5;
  const int cb0 = c * nblk;
  const int cb1 = nblocks < cb0 + nblk ? nblocks : cb0 + nblk;
  c0 = 32 * cb0;
  c1 = n < 32 * cb1 ? n : 32 * cb1;
}

// Weight-gradient items: columns per lane QN and 16-wide rank blocks KB of a
// rank, and the hidden columns one item owns.
__host__ __device__ constexpr int wgrad_qn(int kb) { return kb <= 4 ? 4 : 2; }
__host__ __device__ inline int wgrad_kb(int rank) {
  const int k = (rank + 15) >> 4;
  return k <= 1 ? 1 : (k <= 2 ? 2 : (k <= 4 ? 4 : 8));
}
__host__ __device__ inline int wgrad_cw(int rank) { return 4 * 16 * wgrad_qn(wgrad_kb(rank)); }

// Device-side planning of a request-order batch (lora_sgmv_fused_graph): a
// stable counting sort of the token ids into per-adapter segments, their
// 32-token tiles, and the launch id of the call.
constexpr int kMaxGraphAdapters = 256;
constexpr int kPlanThreads = 1024;
struct DevPlanArgs {
  const int32_t* ids;       // DEVICE [T] adapter id per token (request order)
  const uint64_t* A_ptrs;   // DEVICE [N]
  const uint64_t* B_ptrs;   // DEVICE [N]
  const int32_t* ranks;     // DEVICE [N]
  const float* scales;      // DEVICE [N]
  int32_t* perm;            // [T] sorted position -> request row (adapter order, request order within)
  DevTile* tiles;           // [max_tiles]
  int32_t* count;           // [1] tiles written
  uint64_t* epoch;          // the workspace epoch's slots: each advanced by kEpochCall by every plan
  int32_t T;
  int32_t N;
  int32_t max_rank;         // adapters whose rank is outside [1, max_rank] are skipped
  int32_t max_tiles;
};

// Weight-gradient launch: items are (job, kind, column chunk); a job is one
// adapter (or part of its segments) whose token reduction the item owns.
struct WgradPlan {
  const uint16_t* x;  // bf16 rows (dA operand)
  int64_t ldx;
  const uint16_t* dy;  // bf16 rows (dB operand)
  int64_t lddy;
  const float* U;  // fp32 [T, ldu] sorted positions (dB operand)
  int64_t ldu;
  const float* dU;  // fp32 [T, lddu] sorted positions (dA operand)
  int64_t lddu;
  const uint64_t* dA_tab;  // per adapter fp32 [r, h_in]
  const uint64_t* dB_tab;  // per adapter fp32 [h_out, r]
  const int32_t* token_rows;
  int32_t h_in;
  int32_t h_out;
  int32_t n_jobs;
  int32_t job_item0[kMaxJobs + 1];  // first item of each job (items: dB chunks, then dA chunks); [n_jobs] = total
  int32_t job_nsteps[kMaxJobs];     // 32-token steps over the job's segments
  int32_t job_adapter[kMaxJobs];
  int32_t job_seg0[kMaxJobs];
  int32_t job_nseg[kMaxJobs];
  int32_t job_accum[kMaxJobs];
  float job_scale[kMaxJobs];
  int32_t job_rank[kMaxJobs];
  int32_t job_part[kMaxJobs];  // -1: write the adapter's gradients; else partial slot index
  int32_t seg_tok0[kMaxJobSeg];
  int32_t seg_ntok[kMaxJobSeg];
  float* part_base;     // partial slots: slot s = dB part [h_out][r] then dA part [r][h_in]
  int64_t part_stride;  // floats per slot
};

// Sum of the token-range parts of split weight-gradient jobs: for adapter
// red_adapter[j], its gradients (dB then dA, flattened) become
// (accumulate ? old : 0) + sum of slots red_slot0[j] .. red_slot0[j] + red_nparts[j] - 1,
// added in slot order.
struct WgradReducePlan {
  const float* part_base;
  int64_t part_stride;
  const uint64_t* dA_tab;
  const uint64_t* dB_tab;
  int32_t h_in;
  int32_t h_out;
  int32_t n_red;
  int32_t accumulate;
  int32_t red_item0[kMaxJobs + 1];  // first workgroup of each adapter; [n_red] = grid
  int32_t red_adapter[kMaxJobs];
  int32_t red_rank[kMaxJobs];
  int32_t red_slot0[kMaxJobs];
  int32_t red_nparts[kMaxJobs];
};
constexpr int kReduceElems = 4 * kThreads;  // floats per reduce workgroup

// Transposed copies of the adapter weights for the backward du/dx pass.
struct TransposePlan {
  const uint64_t* A_tab;  // per adapter bf16 [r, h_in]
  const uint64_t* B_tab;  // per adapter bf16 [h_out, r]
  uint16_t* Bt;           // slot s: [r, h_out] at Bt + s * bt_slot_elems
  uint16_t* At;           // slot s: [h_in, round_up(r, 8)] at At + s * at_slot_elems
  int64_t bt_slot_elems;
  int64_t at_slot_elems;
  int32_t h_in;
  int32_t h_out;
  int32_t n_slots;
  int32_t tiles_b;  // 64x64 tiles per slot for B: ceil(h_out/64) * tb_cols
  int32_t tiles_a;  // 64x64 tiles per slot for A: ceil(r8_max/64) * ta_cols
  int32_t tb_cols;  // ceil(r_max/64)
  int32_t ta_cols;  // ceil(h_in/64)
  int32_t slot_adapter[kMaxJobs];
  int32_t slot_rank[kMaxJobs];
};

}  // namespace lora
