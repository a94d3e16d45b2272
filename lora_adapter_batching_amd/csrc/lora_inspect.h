/*
 * lora_inspect.h -- host-only inspection of the launch plans of
 * liblora_sgmv.so. Internal: not part of the public ABI (include/lora_sgmv.h);
 * the test suite uses it to check the segment scheduler on the CPU.
 *
 * lora_inspect_plan() runs the planner of one public call (the same code the
 * call runs, with stand-in device addresses that are never dereferenced)
 * and lists every workgroup of every launch the call would make, without
 * touching a GPU. The scheduler balances segments of heterogeneous ranks and
 * lengths across the compute units ("Technische Samenvatting: PLoRA"
 * (gist.science), "Kernelontwerp": load balancing over heterogeneous
 * adapters), and the listing lets a test check coverage, ownership and
 * balance of that plan.
 */
#ifndef LORA_INSPECT_H
#define LORA_INSPECT_H

#include <stdint.h>

#include "../../include/lora_sgmv.h"

#ifdef __cplusplus
extern "C" {
#endif

enum {
  LORA_PHASE_FWD = 0,
  LORA_PHASE_WGRAD = 1,
  LORA_PHASE_REDUCE = 2,
  LORA_PHASE_TRANSPOSE = 3,
  LORA_PHASE_PLAN = 4 /* device planning of a graph call (one workgroup) */
};

/* Options of lora_inspect_plan(). */
#define LORA_INSPECT_WITH_U 1u     /* fused: u_save given; backward: u given (else recomputed) */
#define LORA_INSPECT_WITH_DX 2u    /* backward: dx given */
#define LORA_INSPECT_ACCUMULATE 4u /* backward: LORA_GRAD_ACCUMULATE */

/* One workgroup of one launch. */
typedef struct lora_plan_item_t {
  int32_t launch;  /* index of the launch, in enqueue order */
  int32_t phase;   /* LORA_PHASE_* */
  int32_t block;   /* workgroup index within the launch */
  int32_t grid;    /* workgroups of the launch */
  int32_t mode;    /* forward: launch mode (0 shrink, 1 expand, 2 on-chip fused, 3 split fused) */
  int32_t kind;    /* forward: -1 idle, 0 shrink part, 1 expand, 2 fused tile, 3 expand after parts;
                      weight gradients: 0 dB, 1 dA; reduce: 0 */
  int32_t tile;    /* forward: tile index; weight gradients: job index; else -1 */
  int32_t adapter; /* adapter of the item (-1 idle) */
  int32_t proj;    /* forward: projection; else 0 */
  int32_t rank;
  int32_t tok0;    /* forward: first sorted position; weight gradients: first entry in ranges */
  int32_t ntok;    /* forward: positions of the tile; weight gradients: number of ranges */
  int32_t lo, hi;  /* forward shrink: k range; forward expand kinds, weight gradients: column range;
                      reduce: flattened element range (dB then dA) */
  int32_t part;    /* weight gradients: partial slot (-1: writes the adapter); reduce: first slot;
                      forward: k-chunks per tile */
  int32_t aux;     /* weight gradients: accumulate flag; reduce: parts; forward: column chunks per tile */
} lora_plan_item_t;

/*
 * op: LORA_OP_SHRINK / EXPAND / FUSED / BACKWARD. num_proj > 1 (FUSED only)
 * plans lora_sgmv_fused_multi over adapters[0..num_proj). cus / xccs: the
 * device the plan is made for (compute units, XCDs). items: room for
 * items_cap records; ranges: room for ranges_cap (first position, count)
 * pairs of weight-gradient token ranges. *n_items / *n_ranges receive the
 * full counts even when they exceed the capacities (records past a capacity
 * are not written). Validation and errors as for the planned call.
 */
int lora_inspect_plan(int op, int32_t num_proj, const lora_adapters_t* const* adapters,
                      const lora_segments_t* segments, uint32_t options, int32_t cus, int32_t xccs,
                      lora_plan_item_t* items, int64_t items_cap, int64_t* n_items, int32_t* ranges,
                      int64_t ranges_cap, int64_t* n_ranges);

/* The workgroups of a device-planned call (lora_sgmv_fused_graph) over
 * num_tokens ids whose batch has `tiles` 32-token tiles: the launch the call
 * makes (for up to 1024 tokens, the fused launch with the item each
 * workgroup picks once it has counted the tiles; above, the plan kernel and
 * then the fused launch). Items carry launch, phase, block, grid, mode,
 * kind, tile and the k range (shrink parts) or column range (expands);
 * adapter, tok0 and ntok are -1 (they depend on the ids). The adapter
 * tables are never dereferenced. Host only. */
int lora_inspect_graph(const lora_graph_adapters_t* adapters, int32_t num_tokens, int32_t tiles, int32_t cus,
                       int32_t xccs, lora_plan_item_t* items, int64_t items_cap, int64_t* n_items);

#ifdef __cplusplus
}
#endif

#endif /* LORA_INSPECT_H */
