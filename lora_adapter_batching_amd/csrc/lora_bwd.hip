// lora_bwd.hip -- packed-training backward kernels for gfx950: transposed
// weight copies for the du/dx pass, and the adapter weight gradients.
//
// The weight gradients reduce over every token of an adapter:
//   dB_i[j][k] = s_i sum_t dy[t][j] u[t][k],   dA_i[k][d] = sum_t du[t][k] x[t][d].
// Each workgroup owns a block of hidden columns of one adapter's gradient and
// walks all of that adapter's tokens, so the reduction is deterministic and
// needs no atomics; tiles follow the hidden dimension, not the rank
// ("Technische Samenvatting: PLoRA" (gist.science), "Kernelontwerp").
#include "lora_device.h"
#include "lora_plan.h"

namespace lora {

// ---------------------------------------------------------------------------
// Transposed copies: Bt_s = B_i^T [r, h_out]; At_s = A_i^T [h_in, round_up(r,8)]
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void transpose_kernel(TransposePlan P) {
  __shared__ alignas(16) uint16_t tile[64][64 + 8];
  const int per = P.tiles_b + P.tiles_a;
  const int s = blockIdx.x / per;
  const int w0 = blockIdx.x - s * per;
  const bool is_b = w0 < P.tiles_b;
  const int w = is_b ? w0 : w0 - P.tiles_b;
  const int r = P.slot_rank[s];
  const int a = P.slot_adapter[s];
  const int r8 = (r + 7) & ~7;
  // source S [rows, cols] (row stride lds); destination D = S^T [cols, rows_pad]
  const uint16_t* src;
  uint16_t* dst;
  int rows, cols, lds, ldd, rows_pad, tcols;
  if (is_b) {  // B_i [h_out, r] -> Bt [r, h_out]
    src = reinterpret_cast<const uint16_t*>(P.B_tab[a]);
    rows = P.h_out; cols = r; lds = r;
    dst = P.Bt + (int64_t)s * P.bt_slot_elems; ldd = P.h_out; rows_pad = P.h_out;
    tcols = P.tb_cols;
  } else {     // A_i [r, h_in] -> At [h_in, r8], columns r..r8-1 zero
    src = reinterpret_cast<const uint16_t*>(P.A_tab[a]);
    rows = r; cols = P.h_in; lds = P.h_in;
    dst = P.At + (int64_t)s * P.at_slot_elems; ldd = r8; rows_pad = r8;
    tcols = P.ta_cols;
  }
  const int r0 = (w / tcols) * 64, c0 = (w % tcols) * 64;
  if (r0 >= rows_pad || c0 >= cols) return;
  // loads: 16 bytes (8 elements of one row) per thread and pass when the
  // source rows are 16-byte aligned (lds a multiple of 8; the base is by
  // contract), else element by element
  if ((lds & 7) == 0) {
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int e = threadIdx.x + kThreads * pass;  // 512 pieces of 8 elements
      const int i = e >> 3, j = (e & 7) * 8;
      const int sr = r0 + i, sc = c0 + j;
      u32x4v v = {0u, 0u, 0u, 0u};
      if (sr < rows && sc < cols)  // cols is a multiple of 8 here, so all 8 are in range
        v = *reinterpret_cast<const u32x4v*>(src + (int64_t)sr * lds + sc);
      *reinterpret_cast<u32x4v*>(&tile[i][j]) = v;
    }
  } else {
    for (int e = threadIdx.x; e < 64 * 64; e += kThreads) {
      const int i = e >> 6, j = e & 63;
      const int sr = r0 + i, sc = c0 + j;
      tile[i][j] = (sr < rows && sc < cols) ? src[(int64_t)sr * lds + sc] : (uint16_t)0;
    }
  }
  __syncthreads();
  // stores: 16 bytes of one destination row per thread and pass (ldd and
  // rows_pad are multiples of 8, so a piece is either whole or outside)
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int e = threadIdx.x + kThreads * pass;
    const int i = e >> 3, j = (e & 7) * 8;  // destination row c0 + i, columns r0 + j .. + 7
    const int dr = c0 + i, dc = r0 + j;
    if (dr < cols && dc < rows_pad) {
      uint32_t q[4];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        q[h] = (uint32_t)tile[j + 2 * h][i] | ((uint32_t)tile[j + 2 * h + 1][i] << 16);
      typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
      *reinterpret_cast<u32x4v*>(dst + (int64_t)dr * ldd + dc) = u32x4v{q[0], q[1], q[2], q[3]};
    }
  }
}

hipError_t launch_transpose(const TransposePlan& P, hipStream_t stream) {
  hipLaunchKernelGGL(transpose_kernel, dim3(P.n_slots * (P.tiles_b + P.tiles_a)), dim3(kThreads),
                     0, stream, P);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weight gradients
// ---------------------------------------------------------------------------
// Both gradients have the form O[j][k] = s * sum_t Z[t][j] Q[t][k] over the
// adapter's tokens t: Z = dy, Q = u for dB (O = dB_i[j][k]); Z = x, Q = du for
// dA (O = dA_i^T, stored as dA_i[k][j]). An item owns 64*QN columns j of one
// adapter's O and reduces over all of the adapter's tokens in steps of 32.
// v_mfma_f32_16x16x32_bf16 takes A = Z^T (16 columns x 32 tokens; each lane
// loads 8 token rows of QN columns and transposes them in registers) and
// B = Q (32 tokens x 16 ranks, fp32 split into bf16 hi + lo, staged through
// LDS transposed). The loads of the next kWgDepth-1 steps are in flight while
// a step is computed.
// Columns per lane QN and rank blocks of 16 (KB) for a rank: wgrad_qn,
// wgrad_kb, wgrad_cw (shared with the host planner).

constexpr int kQtLd = 36;    // LDS row length (floats) of the transposed Q tile
constexpr int kWgDepth = 3;  // steps whose loads are in flight (and LDS Q buffers)

// One 32-token step of an item: the token range and how to address it.
struct WgCursor {
  int seg;   // segment index in the plan (>= seg_end: past the item's tokens)
  int t0;    // first sorted position of the step
  int tend;  // end of the segment
};

template <int KB, int QN>
struct WgRegs {
  uint32_t z[8][QN / 2];  // Z rows 8g + e, this lane's QN columns (bf16 pairs)
  float q[2 * KB];        // this thread's share of the step's Q tile
};

__device__ __forceinline__ void wg_advance(const WgradPlan& P, int seg_end, WgCursor& c) {
  c.t0 += 32;
  while (c.t0 >= c.tend && c.seg < seg_end) {
    ++c.seg;
    if (c.seg < seg_end) {
      c.t0 = P.seg_tok0[c.seg];
      c.tend = c.t0 + P.seg_ntok[c.seg];
    }
  }
}

template <int KB, int QN, bool GATHER>
__device__ __forceinline__ void wg_load(const WgradPlan& P, const uint16_t* Z, int64_t ldz, int ncols,
                                        const float* Q, int64_t ldq, int rank, int ccol, bool col_ok,
                                        int seg_end, const WgCursor& c, WgRegs<KB, QN>& R) {
  const int lane = threadIdx.x & 63, g = lane >> 4;
  const bool live = c.seg < seg_end;
  const int cnt = live ? min(32, c.tend - c.t0) : 0;  // valid tokens of the step (uniform)
  // Z (x or dy) is read by this workgroup alone, once: non-temporal loads
  // (with the streamed dy of the dU/dX pass, the packed-training backward
  // went from 550 to 539 us).
  // Z: a resource over the step's rows (contiguous positions) or over the
  // whole matrix (token_rows gather: a row is read only if it lies wholly
  // inside the resource, with its offset kept in 64 bits)
  __amdgpu_buffer_rsrc_t zr, rr;
  if constexpr (GATHER) {
    zr = mk_rsrc(Z, cnt > 0 ? kGatherSpan : 0);
    rr = mk_rsrc(P.token_rows + (live ? c.t0 : 0), (int64_t)cnt * 4);
  } else {
    zr = mk_rsrc(Z + (int64_t)(live ? c.t0 : 0) * ldz, cnt > 0 ? ((int64_t)(cnt - 1) * ldz + ncols) * 2 : 0);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = 8 * g + e;
    const bool ok = col_ok && r < cnt;
    bool in = ok;
    int64_t row_bytes = (int64_t)r * ldz * 2;
    if constexpr (GATHER) {
      const int32_t row = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rr, ok ? 4 * r : (int)kOff, 0, 0);
      row_bytes = (int64_t)row * ldz * 2;
      in = ok && row_bytes >= 0 && row_bytes <= kGatherSpan - (int64_t)ncols * 2;
    }
    const uint32_t off = in ? (uint32_t)(row_bytes + (int64_t)ccol * 2) : kOff;
    if constexpr (QN == 4) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(zr, (int)off, 0, kNT);
      R.z[e][0] = v[0];
      R.z[e][1] = v[1];
    } else {
      R.z[e][0] = __builtin_amdgcn_raw_buffer_load_b32(zr, (int)off, 0, kNT);
    }
  }
  // Q (fp32, sorted positions): element (tt, k) = (e2 / 16KB, e2 % 16KB)
  const __amdgpu_buffer_rsrc_t qr = mk_rsrc(Q + (int64_t)(live ? c.t0 : 0) * ldq, (int64_t)cnt * ldq * 4);
#pragma unroll
  for (int j = 0; j < 2 * KB; ++j) {
    const int e2 = threadIdx.x + kThreads * j;
    const int tt = e2 / (16 * KB), k = e2 - tt * (16 * KB);
    const uint32_t off = (tt < cnt && k < rank) ? (uint32_t)(((int64_t)tt * ldq + k) * 4) : kOff;
    R.q[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(qr, (int)off, 0, 0));
  }
}

template <int KB, int QN>
__device__ __forceinline__ void wg_commit_q(const WgRegs<KB, QN>& R, float (*Qt)[kQtLd]) {
#pragma unroll
  for (int j = 0; j < 2 * KB; ++j) {
    const int e2 = threadIdx.x + kThreads * j;
    const int tt = e2 / (16 * KB), k = e2 - tt * (16 * KB);
    Qt[k][tt] = R.q[j];
  }
}

template <int KB, int QN>
__device__ __forceinline__ void wg_compute(const WgRegs<KB, QN>& R, float (*Qt)[kQtLd], f32x4 (&acc)[QN][KB]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
  // A operand: frag q = Z[8g + e][column q], e = 0..7 (register transpose)
  bf16x8 fa[QN];
#pragma unroll
  for (int q = 0; q < QN; ++q) {
    u32x4 v;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t lo = R.z[2 * d][q >> 1], hi = R.z[2 * d + 1][q >> 1];
      v[d] = (q & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    fa[q] = as_bf16x8(v);
  }
  // B operand: Q[8g + e][16kb + cl] as bf16 hi + lo
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    float f[8];
    const f32x4 q0 = *reinterpret_cast<const f32x4*>(&Qt[16 * kb + cl][8 * g]);
    const f32x4 q1 = *reinterpret_cast<const f32x4*>(&Qt[16 * kb + cl][8 * g + 4]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = q0[e];
      f[4 + e] = q1[e];
    }
    bf16x8 qh, ql;
    split8(f, qh, ql);
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      acc[q][kb] = mfma16(fa[q], qh, acc[q][kb]);
      acc[q][kb] = mfma16(fa[q], ql, acc[q][kb]);
    }
  }
}

template <int KB, int QN, bool GATHER>
__device__ __forceinline__ void wgrad_item(const WgradPlan& P, int job, int kind, int chunk,
                                           float (*Qt)[128][kQtLd]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, cl = lane & 15;
  const int a = P.job_adapter[job];
  const int rank = P.job_rank[job];
  const bool is_db = kind == 0;
  float* out = reinterpret_cast<float*>(is_db ? P.dB_tab[a] : P.dA_tab[a]);
  if (!out) return;  // whole workgroup: uniform
  // a token-range part of a split job writes its own slot (summed later)
  const int part = P.job_part[job];
  if (part >= 0) out = P.part_base + (int64_t)part * P.part_stride + (is_db ? 0 : (int64_t)P.h_out * rank);
  const uint16_t* Z = is_db ? P.dy : P.x;
  const int64_t ldz = is_db ? P.lddy : P.ldx;
  const float* Q = is_db ? P.U : P.dU;
  const int64_t ldq = is_db ? P.ldu : P.lddu;
  const int ncols = is_db ? P.h_out : P.h_in;
  const float oscale = is_db ? P.job_scale[job] : 1.f;
  const int c0 = chunk * (4 * 16 * QN) + wave * (16 * QN);  // this wave's first column
  const int ccol = c0 + QN * cl;                             // this lane's first column
  const bool col_ok = ccol < ncols;

  f32x4 acc[QN][KB];
#pragma unroll
  for (int q = 0; q < QN; ++q)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) acc[q][kb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int seg0 = P.job_seg0[job];
  const int seg_end = seg0 + P.job_nseg[job];
  const int nsteps = P.job_nsteps[job];
  WgCursor lc{seg0, 0, 0};
  if (seg0 < seg_end) {
    lc.t0 = P.seg_tok0[seg0];
    lc.tend = lc.t0 + P.seg_ntok[seg0];
    if (lc.t0 >= lc.tend) {  // skip empty segments
      lc.t0 -= 32;
      wg_advance(P, seg_end, lc);
    }
  }
  // Ring of D register sets; step i uses set i % D and LDS buffer i % D.
  // The step count is rounded up to a multiple of D: steps past the item's
  // tokens load nothing (all offsets fall outside their resources) and add
  // zeros, so every pass of the loop issues the same loads and each wait
  // covers only the set it needs.
  // (a gathered batch waits for its row indices anyway: a shallow ring)
  constexpr int D = GATHER ? 2 : kWgDepth;
  WgRegs<KB, QN> R[D];
#pragma unroll
  for (int s = 0; s < D; ++s) {
    wg_load<KB, QN, GATHER>(P, Z, ldz, ncols, Q, ldq, rank, ccol, col_ok, seg_end, lc, R[s]);
    wg_advance(P, seg_end, lc);
  }
  for (int i = 0; i < nsteps; i += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      wg_commit_q<KB, QN>(R[s], Qt[s]);
      __syncthreads();
      wg_compute<KB, QN>(R[s], Qt[s], acc);
      wg_load<KB, QN, GATHER>(P, Z, ldz, ncols, Q, ldq, rank, ccol, col_ok, seg_end, lc, R[s]);
      wg_advance(P, seg_end, lc);
    }
  }
  // lane holds C[m = 4g + i][n = cl] of block (q, kb): column c0 + QN*m + q
  // (the A-operand row m came from lane m's columns), rank 16kb + cl
  const bool accum = part < 0 && P.job_accum[job] != 0;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int k = 16 * kb + cl;
    if (k >= rank) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      const int cb = c0 + QN * m;
      if (cb >= ncols) continue;
      float v[QN];
#pragma unroll
      for (int q = 0; q < QN; ++q) v[q] = oscale * acc[q][kb][i];
      if (is_db) {
        // dB_i [h_out][r]: lanes cl write consecutive ranks of one column
        float* o = out + (int64_t)cb * rank + k;
        if (accum) {
#pragma unroll
          for (int q = 0; q < QN; ++q) o[(int64_t)q * rank] += v[q];
        } else {
#pragma unroll
          for (int q = 0; q < QN; ++q) o[(int64_t)q * rank] = v[q];
        }
      } else {
        // dA_i [r][h_in]: the lane's QN columns are contiguous
        float* o = out + (int64_t)k * ncols + cb;
        if constexpr (QN == 4) {
          f32x4 w = f32x4{v[0], v[1], v[2], v[3]};
          if (accum) w += *reinterpret_cast<const f32x4*>(o);
          *reinterpret_cast<f32x4*>(o) = w;
        } else {
#pragma unroll
          for (int q = 0; q < QN; ++q) o[q] = accum ? o[q] + v[q] : v[q];
        }
      }
    }
  }
}

template <bool GATHER>
__global__ __launch_bounds__(kThreads, 2) void wgrad_kernel(WgradPlan P) {
  __shared__ alignas(16) float Qt[kWgDepth][128][kQtLd];
  __shared__ int job_of_item;
  // locate the job with one parallel read of the item table (thread j checks
  // job j); items are laid out job by job, dB chunks before dA chunks
  const int item = blockIdx.x;
  {
    const int j = min((int)threadIdx.x, kMaxJobs - 1);
    const int i0 = P.job_item0[j], i1 = P.job_item0[j + 1];
    if ((int)threadIdx.x < P.n_jobs && item >= i0 && item < i1) job_of_item = j;
  }
  __syncthreads();
  const int job = __builtin_amdgcn_readfirstlane(job_of_item);
  const int cw = wgrad_cw(P.job_rank[job]);
  const int nb_db = (P.h_out + cw - 1) / cw;
  const int local = item - P.job_item0[job];
  const int kind = local < nb_db ? 0 : 1;
  const int chunk = kind == 0 ? local : local - nb_db;
  switch (wgrad_kb(P.job_rank[job])) {
    case 1: wgrad_item<1, wgrad_qn(1), GATHER>(P, job, kind, chunk, Qt); break;
    case 2: wgrad_item<2, wgrad_qn(2), GATHER>(P, job, kind, chunk, Qt); break;
    case 4: wgrad_item<4, wgrad_qn(4), GATHER>(P, job, kind, chunk, Qt); break;
    default: wgrad_item<8, wgrad_qn(8), GATHER>(P, job, kind, chunk, Qt); break;
  }
}

// Sum of split jobs' parts: workgroup w of adapter j takes kReduceElems
// consecutive floats of the adapter's flattened gradients (dB [h_out][r],
// then dA [r][h_in]); both sizes are multiples of 8 floats, so a thread's 4
// floats never straddle the two. The parts are added in slot order.
__global__ __launch_bounds__(kThreads) void wgrad_reduce_kernel(WgradReducePlan R) {
  __shared__ int red_of_item;
  const int item = blockIdx.x;
  {
    const int j = min((int)threadIdx.x, kMaxJobs - 1);
    if ((int)threadIdx.x < R.n_red && item >= R.red_item0[j] && item < R.red_item0[j + 1]) red_of_item = j;
  }
  __syncthreads();
  const int j = __builtin_amdgcn_readfirstlane(red_of_item);
  const int a = R.red_adapter[j], rank = R.red_rank[j];
  const int64_t n_db = (int64_t)R.h_out * rank, n_all = n_db + (int64_t)R.h_in * rank;
  const int64_t e = (int64_t)(item - R.red_item0[j]) * kReduceElems + 4 * threadIdx.x;
  if (e >= n_all) return;
  float* dst = reinterpret_cast<float*>(e < n_db ? R.dB_tab[a] : R.dA_tab[a]);
  if (!dst) return;
  dst += e < n_db ? e : e - n_db;
  const float* src = R.part_base + (int64_t)R.red_slot0[j] * R.part_stride + e;
  f32x4 sum = *reinterpret_cast<const f32x4*>(src);
  for (int p = 1; p < R.red_nparts[j]; ++p) sum += *reinterpret_cast<const f32x4*>(src + p * R.part_stride);
  if (R.accumulate) sum = *reinterpret_cast<const f32x4*>(dst) + sum;
  *reinterpret_cast<f32x4*>(dst) = sum;
}

hipError_t launch_wgrad_reduce(const WgradReducePlan& R, hipStream_t stream) {
  hipLaunchKernelGGL(wgrad_reduce_kernel, dim3(R.red_item0[R.n_red]), dim3(kThreads), 0, stream, R);
  return hipGetLastError();
}

int wgrad_items_for_rank(int rank, int h_in, int h_out) {
  const int cw = wgrad_cw(rank);
  return (h_out + cw - 1) / cw + (h_in + cw - 1) / cw;
}

hipError_t launch_wgrad(const WgradPlan& P, int grid, hipStream_t stream) {
  if (P.token_rows)
    hipLaunchKernelGGL(wgrad_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, P);
  else
    hipLaunchKernelGGL(wgrad_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, P);
  return hipGetLastError();
}

}  // namespace lora
