// Split / no-split decode kernel, vector-ALU variant (gfx950).
//
// One workgroup per task (row, kv head, page range).  The pages of the task
// are dealt round-robin to the workgroup's waves; a wave reads one whole KV
// page per step with coalesced 16-byte buffer loads (one wave-wide load
// covers 1 KiB, i.e. 64/(d/8) tokens), and keeps PF more pages in flight
// while it computes the current one.  Lane layout after a load: the d/8 lanes of a
// "stream" hold one token row, 8 elements each; a wave holds 64/(d/8)
// streams.  Scores are packed dot products (v_dot2) reduced across the
// stream's lanes with DPP; every stream keeps its own running max / sum /
// unnormalised output (online softmax), so no cross-stream traffic happens
// per page.  Streams are merged inside the wave, waves through LDS, and the
// workgroup writes either the partial state (split paths) or the normalised
// output (no-split path).
//
// Method: PersistentKV summary pages, "Methodology / 1. Native block-table
// decode engine" (GQA over paged KV read through the block table, partial
// online-softmax state per disjoint split, empty splits write neutral state).
#include "lens_plan.h"
#include "split_common.h"

namespace pkv {
namespace {

// One task (row, KV head, page range): stream its pages, then combine the
// waves and write the partial state (or, no-split, the normalised output).
template <int D, int GP, bool BF16, int NW, int PF, int MODE>
__device__ __forceinline__ void valu_task(const SplitArgs& a, Task tk, float (&sm_m)[NW][GP],
                                          float (&sm_l)[NW][GP], float (&sm_o)[NW][GP][D]) {
  constexpr int CPT = D / 8;     // 16-byte chunks per token row
  constexpr int TPI = 64 / CPT;  // tokens per wave-wide 16-byte load
  constexpr int NL = 16 / TPI;   // loads per page (16 tokens per page)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane % CPT;  // chunk: elements [8c, 8c+8)
  const int r = lane / CPT;  // stream: tokens r, r+TPI, ... of each page
  const int hkv = a.num_kv_heads;
  const int G = a.group;  // real heads in the group (<= GP)

  const int row = tk.row, g = tk.g, pb = tk.page_begin;
  const int32_t* bt = a.block_table + int64_t(row) * a.max_pages;
  const int first = pb + wave;  // this wave's pages: first, first + NW, ...
  // Page ids of the first 64 of them; issued before the row length is known.
  int pids = load_page_ids<NW>(bt, a.max_pages, first, 0, lane);
  if constexpr (MODE == kModeNoSplit) {
    tk.tok_end = a.seq_lens[row];
    if (tk.tok_end == 0) {  // empty row: zero output, lse = -inf
      write_empty_row<NW>(a, tk, G, D);
      return;
    }
  }
  const int tok_end = tk.tok_end;
  const int pe = (tok_end + 15) >> 4;

  // ---- query: GP heads x 8 elements per lane ------------------------------
  uint4 qv[GP];
  {
    const uint16_t* qp =
        static_cast<const uint16_t*>(a.q) + (int64_t(row) * a.num_q_heads + g * G) * D + 8 * c;
#pragma unroll
    for (int h = 0; h < GP; ++h) qv[h] = (h < G) ? load16(qp + h * D) : zero4();
  }

  float m[GP], l[GP], o[GP][8];
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[h][j] = 0.f;
  }

  const int64_t page_stride = int64_t(hkv) * 16 * D;  // elements
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k_pool) + int64_t(g) * 16 * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v_pool) + int64_t(g) * 16 * D;
  const float sl2 = a.scale_log2;

  const int cnt = (pe > first) ? (pe - first + NW - 1) / NW : 0;

  // Chunk kc of the wave's pages: pids lane j holds the pool page of page kc + j.
  int kc = 0;

  // Buffer descriptor of the chunk's page j: num_records = bytes of its real
  // tokens, so loads of tokens past N -- and of null pages j >= cnt_c, which
  // pad the ring -- return zeros without touching memory.
  auto page_rsrc = [&](const uint16_t* base, int j, int cnt_c) {
    int nbytes = 0;
    const uint16_t* ptr = base;
    if (j < cnt_c) {
      const int pid = __builtin_amdgcn_readlane(pids, j);
      const int valid = min(16, tok_end - (first + (kc + j) * NW) * 16);
      nbytes = valid * D * 2;
      ptr = base + int64_t(pid) * page_stride;
    }
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(ptr), (short)0, nbytes,
                                             kBufferFlags);
  };
  auto issue = [&](int j, int cnt_c, uint4 (&kk)[NL], uint4 (&vv)[NL]) {
    const auto kr = page_rsrc(kbase, j, cnt_c);
    const auto vr = page_rsrc(vbase, j, cnt_c);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      kk[i] = buffer_load16(kr, lane * 16 + i * 1024);
      vv[i] = buffer_load16(vr, lane * 16 + i * 1024);
    }
  };

  auto compute_page = [&](int j, const uint4 (&kk)[NL], const uint4 (&vv)[NL]) {
    const int valid = tok_end - (first + (kc + j) * NW) * 16;
    float x[NL][GP];
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int h = 0; h < GP; ++h) x[i][h] = group_sum<CPT>(dot8<BF16>(kk[i], qv[h], 0.f)) * sl2;
    float vf[NL][8];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const uint32_t w[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vf[i][2 * j] = Elem<BF16>::lo(w[j]);
        vf[i][2 * j + 1] = Elem<BF16>::hi(w[j]);
      }
    }
    const bool tail = valid < 16;  // wave-uniform
    if (tail) {
#pragma unroll
      for (int i = 0; i < NL; ++i)
        if (i * TPI + r >= valid)
#pragma unroll
          for (int h = 0; h < GP; ++h) x[i][h] = kNegInf;
    }
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      float mp = x[0][h];
#pragma unroll
      for (int i = 1; i < NL; ++i) mp = fmaxf(mp, x[i][h]);
      const float mn = fmaxf(m[h], mp);
      // A stream that has only seen masked tokens keeps m = -inf; use 0 as
      // the exponent base so that exp2(-inf - base) = 0 instead of NaN.
      const float base = (mn == kNegInf) ? 0.f : mn;
      const float alpha = fast_exp2(m[h] - base);
      m[h] = mn;
      float lh = l[h] * alpha;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[h][j] *= alpha;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const float p = fast_exp2(x[i][h] - base);
        lh += p;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[h][j] = fmaf(p, vf[i][j], o[h][j]);
      }
      l[h] = lh;
    }
  };

  // Register ring of R = PF + 1 pages: page j + PF is in flight while page j
  // is computed.  The steady-state loop has no loads under a branch, so the
  // compiler's in-order vmcnt waits keep PF pages outstanding.
  constexpr int R = PF + 1;
  uint4 kb[R][NL], vb[R][NL];
  for (kc = 0; kc < cnt; kc += 64) {
    const int cnt_c = min(64, cnt - kc);
    if (kc > 0) pids = load_page_ids<NW>(bt, a.max_pages, first, kc, lane);
#pragma unroll
    for (int u = 0; u < PF; ++u) issue(u, cnt_c, kb[u], vb[u]);
    for (int j0 = 0; j0 < cnt_c; j0 += R) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int j = j0 + u;
        issue(j + PF, cnt_c, kb[(u + PF) % R], vb[(u + PF) % R]);
        if (j < cnt_c) compute_page(j, kb[u], vb[u]);
      }
    }
  }

  // ---- merge the wave's streams (lanes r = 0 .. TPI-1) ---------------------
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    float mx = m[h];
#pragma unroll
    for (int sh = CPT; sh < 64; sh <<= 1) mx = fmaxf(mx, shfl_xor(mx, sh));
    const float wgt = (m[h] == kNegInf) ? 0.f : fast_exp2(m[h] - mx);
    float lh = l[h] * wgt;
#pragma unroll
    for (int sh = CPT; sh < 64; sh <<= 1) lh += shfl_xor(lh, sh);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v = o[h][j] * wgt;
#pragma unroll
      for (int sh = CPT; sh < 64; sh <<= 1) v += shfl_xor(v, sh);
      o[h][j] = v;
    }
    m[h] = mx;
    l[h] = lh;
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sm_o[wave][h][8 * c + j] = o[h][j];
      if (c == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  // ---- merge the waves and write ------------------------------------------
  combine_waves_and_store<D, GP, NW, BF16, MODE>(a, tk, G, sm_m, sm_l, sm_o);
}

// Grid modes as in the matrix-core kernel: one workgroup per workqueue task /
// bucket slot / (row, KV head), or a persistent grid over a device-built plan
// or over the workqueue each workgroup derives from the device lengths.
template <int D, int GP, bool BF16, int NW, int PF, int MODE>
__global__ __launch_bounds__(NW * 64) void split_valu_kernel(SplitArgs a) {
  __shared__ float sm_m[NW][GP];
  __shared__ float sm_l[NW][GP];
  __shared__ __align__(16) float sm_o[NW][GP][D];
  if constexpr (MODE == kModePersistent) {
    persistent_plan_loop(a, [&](const Task& tk) {
      valu_task<D, GP, BF16, NW, PF, kModeWorkqueue>(a, tk, sm_m, sm_l, sm_o);
    });
  } else if constexpr (MODE == kModeLens) {
    lens_loop<NW * 64>(a, [&](const Task& tk) {
      valu_task<D, GP, BF16, NW, PF, kModeWorkqueue>(a, tk, sm_m, sm_l, sm_o);
    });
  } else {
    const Task tk = decode_task<MODE>(a, launch_item<MODE>(a));
    if constexpr (MODE == kModeBucket) {
      if (tk.empty) {  // empty split: neutral state, exit early
        write_neutral<NW>(a, tk, a.group, D);
        return;
      }
    }
    valu_task<D, GP, BF16, NW, PF, MODE>(a, tk, sm_m, sm_l, sm_o);
  }
}

template <int D, int GP, bool BF16, int NW, int PF>
pkv_status launch_valu_modes(int mode, const SplitArgs& a, int grid, hipStream_t s) {
  const dim3 block(NW * 64);
  if (mode == kModeWorkqueue)
    hipLaunchKernelGGL((split_valu_kernel<D, GP, BF16, NW, PF, kModeWorkqueue>), dim3(grid), block, 0,
                       s, a);
  else if (mode == kModeBucket)
    hipLaunchKernelGGL((split_valu_kernel<D, GP, BF16, NW, PF, kModeBucket>), bucket_grid(a, grid), block, 0, s, a);
  else if (mode == kModeNoSplit)
    hipLaunchKernelGGL((split_valu_kernel<D, GP, BF16, NW, PF, kModeNoSplit>), dim3(grid), block, 0,
                       s, a);
  else if (mode == kModePersistent)
    hipLaunchKernelGGL((split_valu_kernel<D, GP, BF16, NW, PF, kModePersistent>), dim3(grid), block,
                       0, s, a);
  else
    hipLaunchKernelGGL((split_valu_kernel<D, GP, BF16, NW, PF, kModeLens>), dim3(grid), block, 0, s,
                       a);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

template <int D, bool BF16>
pkv_status launch_valu_g(int gp, int mode, const SplitArgs& a, int grid, hipStream_t s) {
  switch (gp) {
    case 1: return launch_valu_modes<D, 1, BF16, 8, 2>(mode, a, grid, s);
    case 2: return launch_valu_modes<D, 2, BF16, 8, 2>(mode, a, grid, s);
    case 4: return launch_valu_modes<D, 4, BF16, 8, 2>(mode, a, grid, s);
    case 8: return launch_valu_modes<D, 8, BF16, 4, 2>(mode, a, grid, s);
    default: return PKV_ESHAPE;
  }
}

}  // namespace

// Group sizes up to 8 run on the vector ALUs with the group padded to the next
// power of two (padded heads get q = 0 and are never written).
pkv_status launch_split_valu(const pkv_problem& p, int mode, const SplitArgs& a, int grid,
                             hipStream_t s) {
  const int G = p.num_q_heads / p.num_kv_heads;
  const int gp = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : 0;
  if (gp == 0) return PKV_ESHAPE;
  const bool bf = p.dtype == PKV_BF16;
  if (p.head_dim == 128)
    return bf ? launch_valu_g<128, true>(gp, mode, a, grid, s)
              : launch_valu_g<128, false>(gp, mode, a, grid, s);
  return bf ? launch_valu_g<64, true>(gp, mode, a, grid, s)
            : launch_valu_g<64, false>(gp, mode, a, grid, s);
}

}  // namespace pkv
