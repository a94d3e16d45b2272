// lora_plan.h -- launch plans shared by the host planner and the gfx950
// kernels of the multi-adapter LoRA library. Internal; not part of the ABI.
//
// A plan travels by value as the kernel argument, so a call needs no
// host-to-device copy of metadata: segment tables live in the kernel-argument
// segment and are read with scalar loads.
#pragma once
#include <stdint.h>

namespace lora {

constexpr int kThreads = 256;  // 4 wave64 per workgroup
constexpr int kTileM = 32;     // tokens per tile (the N side of a 32x32 MFMA)
constexpr int kMaxSeg = 128;   // segments per forward launch
constexpr int kMaxJobs = 64;   // adapter jobs per weight-gradient launch
constexpr int kMaxJobSeg = 128;
constexpr int kMaxPartials = 2048;  // (tile, k-chunk) parts in split modes (bounds the workspace)
constexpr int kMaxProj = 4;         // projections over one x in one fused launch

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
// follow at byte offset kStampOffset (one uint64 per (tile, k-chunk)).
constexpr int kCtrTiles = 64;        // per-tile arrival counters start here
constexpr int kStampOffset = 4096;   // bytes from the counters to the stamps

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
  float* partials;            // split-K partial sums [tile][ks][32][rpad]
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
