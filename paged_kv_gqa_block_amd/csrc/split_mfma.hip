// Split / no-split decode kernel, matrix-core variant (gfx950, d = 128).
//
// Same task decomposition, page ring and buffer-descriptor loads as the
// vector-ALU kernel (split_valu.hip); the difference is the P*V product.
//
// Lane layout after one page is loaded (coalesced 16-byte loads): lane l holds
// tokens kg, kg+4, kg+8, kg+12 of the page (kg = l / 16) and elements
// [8c, 8c+8) of each (c = l % 16).
//
//  * Scores run on v_mfma_f32_16x16x32: A = K [16 tokens x 32 elements],
//    B = Q^T [32 elements x 16 heads (padded)], D = S [16 tokens x 16 heads].
//    MFMA operands want one token per lane column, the transpose of the
//    coalesced layout, so each wave writes its K page into a private LDS tile
//    (ds_write_b128, rows XOR-swizzled so neither the writes nor the MFMA
//    reads conflict on banks) and reads it back in operand order.  A's row m
//    is token (m / 4) + 4 (m % 4): then the D registers of lane (kg, c) are the
//    scores of head c for tokens kg + 4r -- the lane's own tokens.
//  * Softmax uses one running max per query head for the whole wave: lane
//    (kg, c) owns head c and reduces the page max over the 4 row groups with
//    cross-row lane swaps.
//  * P*V runs on v_mfma_f32_16x16x16: A = P [16 heads x 16 tokens],
//    B = V [16 tokens x 16 output elements], D = O [16 heads x 16 elements].
//    Token slot k = 4*kg + i is token kg + 4i, which is what lane (n, kg)
//    holds in V load i, so B needs only byte permutes: MFMA j (0..7) covers
//    output elements 8n + j.  A is the lane's own p values for head c, split
//    into a 16-bit high part and a 16-bit residual so the product keeps
//    fp32-level precision in P.
//  * O is rescaled only when some head's running max grew (wave-uniform
//    test), which after the first pages is rare.
//
// Method: PersistentKV summary pages, "Methodology / 1. Native block-table
// decode engine" (GQA over paged KV read through the block table, partial
// online-softmax state per disjoint split, empty splits write neutral state).
#include "lens_plan.h"
#include "split_common.h"

namespace pkv {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// 16 x 16 x 32 score product (A = K rows, B = Q^T columns).
template <bool BF16>
__device__ __forceinline__ float4_t mfma_qk(const uint4& a, const uint4& b, float4_t c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

// Physical 16-byte chunk of (token t, chunk ch) inside a 256-byte K-tile row.
// The XOR key maps the 16 tokens the MFMA reads together onto 16 distinct
// chunk positions.
__device__ __forceinline__ int ktile_chunk(int t, int ch) {
  return ch ^ (((t & 3) << 2) | (t >> 2));
}

// Cross-row reductions with the gfx950 row-swap instructions.  With both
// operands equal to x, the two results of a swap hold, in every lane l, the
// values of lanes l and l ^ 16 (permlane16) or l and l ^ 32 (permlane32), in
// some order; combining them with a symmetric op reduces across the rows.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// P operands.  P is split into a 16-bit high part and the 16-bit rounding of
// its residual, P ~= hi + lo with about 22 (fp16) or 16 (bf16) significant
// bits; both parts go through the matrix core, so the product keeps
// fp32-level precision in P.
template <bool BF16>
struct Pv;

template <>
struct Pv<false> {  // fp16 P and V
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    const half2_t h = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    return __builtin_bit_cast(uint32_t, h);
  }
  static __device__ __forceinline__ float lo(uint32_t w) { return Elem<false>::lo(w); }
  static __device__ __forceinline__ float hi(uint32_t w) { return Elem<false>::hi(w); }
  static __device__ __forceinline__ float4_t mfma(uint2 a, uint2 b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, a),
                                                 __builtin_bit_cast(half4_t, b), c, 0, 0, 0);
  }
};

template <>
struct Pv<true> {  // bf16 P and V
  // One v_cvt_pk_bf16_f32 (gfx950): both values rounded to nearest even, the
  // default rounding mode.  P is finite, so no NaN handling is needed here.
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef float float2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{a, b}, bf162_t));
  }
  static __device__ __forceinline__ float lo(uint32_t w) { return Elem<true>::lo(w); }
  static __device__ __forceinline__ float hi(uint32_t w) { return Elem<true>::hi(w); }
  static __device__ __forceinline__ float4_t mfma(uint2 a, uint2 b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, a),
                                                     __builtin_bit_cast(bf16x4_t, b), c, 0, 0, 0);
  }
};

// LDS of one workgroup: the waves' partial states and each wave's K tile.
template <int GP, int NW>
struct MfmaShared {
  float m[NW][GP];
  float l[NW][GP];
  alignas(16) float o[NW][GP][128];
  uint4 k[NW][16][16];  // per-wave K tile: [token][physical chunk]
};

// One task (row, KV head, page range): stream its pages, then combine the
// waves and write the partial state (or, no-split, the normalised output).
template <int GP, bool BF16, int NW, int PF, int MODE>
__device__ __forceinline__ void mfma_task(const SplitArgs& a, Task tk, MfmaShared<GP, NW>& sh) {
  constexpr int D = 128;
  constexpr int NL = 4;      // 16-byte loads per page per pool (4 tokens each)
  constexpr int HR = (GP + 3) / 4;  // MFMA output row groups holding real heads
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15;   // element chunk [8c, 8c+8); also MFMA column n / head m
  const int kg = lane >> 4;  // row group: tokens kg + 4i
  const int hkv = a.num_kv_heads;
  const int G = a.group;
  auto& sm_m = sh.m;
  auto& sm_l = sh.l;
  auto& sm_o = sh.o;
  auto& sm_k = sh.k;

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

  // B operand of the score MFMAs: lane (kg, c) holds elements
  // [32t + 8kg, 32t + 8kg + 8) of head c for MFMA t (zero for padded heads).
  uint4 qb[4];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (int64_t(row) * a.num_q_heads + g * G + c) * D + 8 * kg;
#pragma unroll
    for (int t = 0; t < 4; ++t) qb[t] = (c < G) ? load16(qp + 32 * t) : zero4();
  }
  // Token read by this lane as MFMA A row m = c.
  const int a_tok = (c >> 2) + 4 * (c & 3);

  // Running max of head c (this lane's softmax head) in log2 units, this
  // lane's share of the sum, and the MFMA accumulators O[j][r]:
  // O[4*kg + r][8*c + j].
  float m_run = kNegInf, l_part = 0.f;
  float4_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t page_stride = int64_t(hkv) * 16 * D;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k_pool) + int64_t(g) * 16 * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v_pool) + int64_t(g) * 16 * D;
  const float sl2 = a.scale_log2;
  const int cnt = (pe > first) ? (pe - first + NW - 1) / NW : 0;

  int kc = 0;
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
    // K page -> LDS tile (token kg + 4i, chunk c), then back in A order.
    uint4 (&tile)[16][16] = sm_k[wave];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int t = kg + 4 * i;
      tile[t][ktile_chunk(t, c)] = kk[i];
    }
    float4_t sacc = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t)
      sacc = mfma_qk<BF16>(tile[a_tok][ktile_chunk(a_tok, 4 * t + kg)], qb[t], sacc);
    // Scores of head c for this lane's tokens kg + 4i, in log2 units.
    float xs[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) xs[i] = sacc[i] * sl2;
    if (valid < 16) {  // tail page: tokens kg + 4i >= valid do not exist
#pragma unroll
      for (int i = 0; i < NL; ++i)
        if (kg + 4 * i >= valid) xs[i] = kNegInf;
    }
    float mp = fmaxf(fmaxf(xs[0], xs[1]), fmaxf(xs[2], xs[3]));
    mp = max_xor32(max_xor16(mp));  // page max of head c over all 16 tokens
    const float mn = fmaxf(m_run, mp);  // finite: every page has a real token
    const bool grew = mn > m_run;
    if (__builtin_amdgcn_ballot_w64(grew) != 0) {  // rescale O and l to the new max
      const float alpha = fast_exp2(m_run - mn);
      l_part *= alpha;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // O row 4*kg + r belongs to head 4*kg + r, whose alpha sits in lane
        // (row 0, column 4*kg + r).
        const float ar = __int_as_float(
            __builtin_amdgcn_ds_bpermute((4 * kg + r) << 2, __float_as_int(alpha)));
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) acc[jj][r] *= ar;
      }
      m_run = mn;
    }
    float p[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      p[i] = fast_exp2(xs[i] - m_run);
      l_part += p[i];
    }
    // B operands: element 8c + jj of tokens kg + 4i, i = 0..3.
    const uint32_t w[NL][4] = {{vv[0].x, vv[0].y, vv[0].z, vv[0].w},
                               {vv[1].x, vv[1].y, vv[1].z, vv[1].w},
                               {vv[2].x, vv[2].y, vv[2].z, vv[2].w},
                               {vv[3].x, vv[3].y, vv[3].z, vv[3].w}};
    using PV = Pv<BF16>;
    const uint2 ph = make_uint2(PV::pack2(p[0], p[1]), PV::pack2(p[2], p[3]));
    const uint2 pl = make_uint2(PV::pack2(p[0] - PV::lo(ph.x), p[1] - PV::hi(ph.x)),
                                PV::pack2(p[2] - PV::lo(ph.y), p[3] - PV::hi(ph.y)));
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const uint32_t sel = (jj & 1) ? 0x07060302u : 0x05040100u;
      const uint2 bv = make_uint2(__builtin_amdgcn_perm(w[1][jj >> 1], w[0][jj >> 1], sel),
                                  __builtin_amdgcn_perm(w[3][jj >> 1], w[2][jj >> 1], sel));
      acc[jj] = PV::mfma(ph, bv, acc[jj]);
      acc[jj] = PV::mfma(pl, bv, acc[jj]);
    }
  };

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

  // ---- wave totals: l summed over the 4 row groups -------------------------
  const float l_tot = sum_xor32(sum_xor16(l_part));
  if (kg < HR) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * kg + r;
      if (h < GP) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) sm_o[wave][h][8 * c + jj] = acc[jj][r];
      }
    }
  }
  if (lane < GP) {
    sm_m[wave][lane] = m_run;  // -inf when the wave had no pages
    sm_l[wave][lane] = l_tot;
  }
  __syncthreads();

  // ---- merge the waves and write ------------------------------------------
  combine_waves_and_store<D, GP, NW, BF16, MODE>(a, tk, G, sm_m, sm_l, sm_o);
}

// Grid modes: one workgroup per workqueue task / bucket slot / (row, KV head);
// or persistent: a fixed grid claiming tasks of a device-built workqueue whose
// task count is read from the plan on the device; or self-planned: the same
// persistent grid over the workqueue each workgroup derives from the device
// lengths in LDS (no plan in memory).
// With one page in flight per wave (PF = 1) the kernel fits in 168 registers
// per lane without spilling, so three waves share each SIMD (three
// workgroups per CU) instead of the two the compiler would otherwise pick.
template <int GP, bool BF16, int NW, int PF, int MODE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(PF == 1 ? 3 : 1, 8)))
void split_mfma_kernel(SplitArgs a) {
  __shared__ MfmaShared<GP, NW> sh;
  if constexpr (MODE == kModePersistent) {
    persistent_plan_loop(a, [&](const Task& tk) {
      mfma_task<GP, BF16, NW, PF, kModeWorkqueue>(a, tk, sh);
    });
  } else if constexpr (MODE == kModeLens) {
    lens_loop<NW * 64>(a, [&](const Task& tk) {
      mfma_task<GP, BF16, NW, PF, kModeWorkqueue>(a, tk, sh);
    });
  } else {
    const Task tk = decode_task<MODE>(a, launch_item<MODE>(a));
    if constexpr (MODE == kModeBucket) {
      if (tk.empty) {  // empty split: neutral state, exit early
        write_neutral<NW>(a, tk, a.group, 128);
        return;
      }
    }
    mfma_task<GP, BF16, NW, PF, MODE>(a, tk, sh);
  }
}

template <int GP, bool BF16, int NW, int PF>
pkv_status launch_mfma_modes(int mode, const SplitArgs& a, int grid, hipStream_t s) {
  const dim3 block(NW * 64);
  if (mode == kModeWorkqueue)
    hipLaunchKernelGGL((split_mfma_kernel<GP, BF16, NW, PF, kModeWorkqueue>), dim3(grid), block, 0,
                       s, a);
  else if (mode == kModeBucket)
    hipLaunchKernelGGL((split_mfma_kernel<GP, BF16, NW, PF, kModeBucket>), bucket_grid(a, grid), block, 0, s, a);
  else if (mode == kModeNoSplit)
    hipLaunchKernelGGL((split_mfma_kernel<GP, BF16, NW, PF, kModeNoSplit>), dim3(grid), block, 0,
                       s, a);
  else if (mode == kModePersistent)
    hipLaunchKernelGGL((split_mfma_kernel<GP, BF16, NW, PF, kModePersistent>), dim3(grid), block,
                       0, s, a);
  else
    hipLaunchKernelGGL((split_mfma_kernel<GP, BF16, NW, PF, kModeLens>), dim3(grid), block, 0, s,
                       a);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

// 4 waves per workgroup with one page in flight per wave (139 registers,
// three waves per SIMD): three workgroups share a CU, so one task's start-up
// overlaps another's streaming.  Measured on MI355X against 8 waves and/or
// two pages in flight: equal on one long row, 5-8 % faster on batched
// workloads; three resident workgroups instead of two: 0.5-2 % faster on
// every workload.
template <bool BF16>
pkv_status launch_mfma_g(int gp, int mode, const SplitArgs& a, int grid, hipStream_t s) {
  switch (gp) {
    case 1: return launch_mfma_modes<1, BF16, 4, 1>(mode, a, grid, s);
    case 2: return launch_mfma_modes<2, BF16, 4, 1>(mode, a, grid, s);
    case 4: return launch_mfma_modes<4, BF16, 4, 1>(mode, a, grid, s);
    case 8: return launch_mfma_modes<8, BF16, 4, 1>(mode, a, grid, s);
    case 16: return launch_mfma_modes<16, BF16, 4, 2>(mode, a, grid, s);
    default: return PKV_ESHAPE;
  }
}

}  // namespace

// d = 128 only; the group is padded to the next power of two (<= 16).
pkv_status launch_split_mfma(const pkv_problem& p, int mode, const SplitArgs& a, int grid,
                             hipStream_t s) {
  if (p.head_dim != 128) return PKV_ESHAPE;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int gp = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : G <= 16 ? 16 : 0;
  if (gp == 0) return PKV_ESHAPE;
  return p.dtype == PKV_BF16 ? launch_mfma_g<true>(gp, mode, a, grid, s)
                             : launch_mfma_g<false>(gp, mode, a, grid, s);
}

}  // namespace pkv
