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
  __shared__ uint16_t tile[64][66];
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
  for (int e = threadIdx.x; e < 64 * 64; e += kThreads) {
    const int i = e >> 6, j = e & 63;
    const int sr = r0 + i, sc = c0 + j;
    tile[i][j] = (sr < rows && sc < cols) ? src[(int64_t)sr * lds + sc] : (uint16_t)0;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += kThreads) {
    const int i = e >> 6, j = e & 63;
    const int dr = c0 + i, dc = r0 + j;
    if (dr < cols && dc < rows_pad) dst[(int64_t)dr * ldd + dc] = tile[j][i];
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
// Columns per lane QN and rank blocks of 16 (KB) for a rank: QN * KB = 16
// keeps 64 fp32 accumulators per lane for every rank.
__host__ __device__ constexpr int wgrad_qn(int kb) { return kb <= 2 ? 8 : (kb == 4 ? 4 : 2); }
__host__ __device__ inline int wgrad_kb(int rank) {
  const int k = (rank + 15) >> 4;
  return k <= 1 ? 1 : (k <= 2 ? 2 : (k <= 4 ? 4 : 8));
}
__host__ __device__ inline int wgrad_cw(int rank) { return 4 * 16 * wgrad_qn(wgrad_kb(rank)); }

constexpr int kQtLd = 36;  // LDS row length (floats) of the transposed u/du tile

template <int QN>
__device__ __forceinline__ void load_row_cols(const uint16_t* p, bool ok, uint32_t (&w)[QN / 2]) {
  if constexpr (QN == 8) {
    const u32x4 v = ok ? ld16(p) : zero16();
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else if constexpr (QN == 4) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = ok ? *reinterpret_cast<const u32x2*>(p) : u32x2{0u, 0u};
    w[0] = v[0]; w[1] = v[1];
  } else {
    w[0] = ok ? *reinterpret_cast<const uint32_t*>(p) : 0u;
  }
}

template <int KB, int QN>
__device__ __forceinline__ void wgrad_item(const WgradPlan& P, int job, int kind, int chunk, float (*Qt)[kQtLd]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, cl = lane & 15;
  const int a = P.job_adapter[job];
  const int rank = P.job_rank[job];
  const bool is_db = kind == 0;
  float* out = reinterpret_cast<float*>(is_db ? P.dB_tab[a] : P.dA_tab[a]);
  if (!out) return;  // whole workgroup: uniform
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

  const int seg0 = P.job_seg0[job], nseg = P.job_nseg[job];
  for (int sgi = 0; sgi < nseg; ++sgi) {
    const int tok0 = P.seg_tok0[seg0 + sgi];
    const int tend = tok0 + P.seg_ntok[seg0 + sgi];
    for (int t0 = tok0; t0 < tend; t0 += 32) {
      // stage Q[t0 .. t0+31][0 .. 16*KB) transposed into LDS
      for (int e = threadIdx.x; e < 32 * 16 * KB; e += kThreads) {
        const int tt = e / (16 * KB), k = e - tt * (16 * KB);
        Qt[k][tt] = (t0 + tt < tend && k < rank) ? Q[(int64_t)(t0 + tt) * ldq + k] : 0.f;
      }
      // Z rows t0 + 8g + e, columns ccol .. ccol+QN-1
      uint32_t w[8][QN / 2];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = t0 + 8 * g + e;
        const bool ok = col_ok && t < tend;
        const int64_t row = ok ? (P.token_rows ? (int64_t)P.token_rows[t] : (int64_t)t) : 0;
        load_row_cols<QN>(Z + row * ldz + ccol, ok, w[e]);
      }
      __syncthreads();
      // A operand: frag q = Z[t0 + 8g + e][ccol + q], e = 0..7 (register transpose)
      bf16x8 fa[QN];
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        u32x4 v;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t lo = w[2 * d][q >> 1], hi = w[2 * d + 1][q >> 1];
          v[d] = (q & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        fa[q] = as_bf16x8(v);
      }
      // B operand: Q[t0 + 8g + e][16kb + cl] as bf16 hi + lo
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = Qt[16 * kb + cl][8 * g + e];
        bf16x8 qh, ql;
        split8(f, qh, ql);
#pragma unroll
        for (int q = 0; q < QN; ++q) {
          acc[q][kb] = mfma16(fa[q], qh, acc[q][kb]);
          acc[q][kb] = mfma16(fa[q], ql, acc[q][kb]);
        }
      }
      __syncthreads();
    }
  }
  // lane holds C[m = 4g + i][n = cl] of block (q, kb): column ccol(m) + q where
  // the A-operand row m came from lane m's columns c0 + QN*m, rank 16kb + cl
  const bool accum = P.job_accum[job] != 0;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int k = 16 * kb + cl;
    if (k >= rank) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      const int cb = c0 + QN * m;
      if (cb >= ncols) continue;
      if (is_db) {
#pragma unroll
        for (int q = 0; q < QN; ++q) {
          float* o = out + (int64_t)(cb + q) * rank + k;
          const float v = oscale * acc[q][kb][i];
          *o = accum ? (*o + v) : v;
        }
      } else {
        float* o = out + (int64_t)k * ncols + cb;
#pragma unroll
        for (int q = 0; q < QN; ++q) {
          const float v = oscale * acc[q][kb][i];
          o[q] = accum ? (o[q] + v) : v;
        }
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void wgrad_kernel(WgradPlan P) {
  __shared__ float Qt[128][kQtLd];
  // locate the job: items are laid out job by job; each job has its own
  // column width (from its rank) and therefore its own item count
  int item = blockIdx.x;
  int job = 0;
  int per = 0, nb_db = 0;
  for (; job < P.n_jobs; ++job) {
    const int cw = wgrad_cw(P.job_rank[job]);
    nb_db = (P.h_out + cw - 1) / cw;
    per = nb_db + (P.h_in + cw - 1) / cw;
    if (item < per) break;
    item -= per;
  }
  if (job >= P.n_jobs) return;
  const int kind = item < nb_db ? 0 : 1;
  const int chunk = kind == 0 ? item : item - nb_db;
  switch (wgrad_kb(P.job_rank[job])) {
    case 1: wgrad_item<1, wgrad_qn(1)>(P, job, kind, chunk, Qt); break;
    case 2: wgrad_item<2, wgrad_qn(2)>(P, job, kind, chunk, Qt); break;
    case 4: wgrad_item<4, wgrad_qn(4)>(P, job, kind, chunk, Qt); break;
    default: wgrad_item<8, wgrad_qn(8)>(P, job, kind, chunk, Qt); break;
  }
}

int wgrad_items_for_rank(int rank, int h_in, int h_out) {
  const int cw = wgrad_cw(rank);
  return (h_out + cw - 1) / cw + (h_in + cw - 1) / cw;
}

hipError_t launch_wgrad(const WgradPlan& P, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(wgrad_kernel, dim3(grid), dim3(kThreads), 0, stream, P);
  return hipGetLastError();
}

}  // namespace lora
