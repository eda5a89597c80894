// Forward launch sequence of the Nystrom path, shared by the per-type
// translation units fwd_f32.hip, fwd_bf16.hip and fwd_bf16x.hip, each of
// which instantiates dispatch_m for its (I/O type, head size) pairs.
//
// Launch sequence for one Nystrom call (all on the caller's stream):
//   1 k_landmark   landmarks Qt, Kt (+ bf16 hi/lo); skipped when the
//                  module's projection has formed them (k_qkv.hpp)
//   2 k_gram       per head A = softmax(Qt Kt^T), its max column / row sum;
//                  only when the pseudo-inverse blocks cannot form A
//                  themselves (m > 128, or the original init with more
//                  heads than can meet in one resident round)
//   3 k_pinv_bv    one launch holding both the per-head pseudo-inverse
//                  blocks (m <= 128) and the B V partial blocks, so the
//                  pseudo-inverse chain runs beside the K/V stream
//     (m > 128, bf16 I/O: A by row blocks in its first blocks at d = 64,
//     k_gram_rows before it at other head sizes, and 3 k_pinv_mm launches
//     per iteration after it; float32 I/O: k_gram, then k_pinv_init and 4
//     k_pinv_gemm launches per iteration after it)
//   4 k_mw         B V from the partials, W = Z (B V) and its operand
//                  fragments
//   5 k_out_stream F W + conv(V) -> out (bf16 I/O; k_out for float32)
// Kernel boundaries are the only cross-workgroup synchronisation, apart
// from the one meeting of the pseudo-inverse blocks for the original init
// (data handed between workgroups of one launch across XCDs would need L2
// write-back and invalidation, which cost far more here than a launch).
#pragma once

#include <cmath>

#include "host.hpp"
#include "k_bv.hpp"
#include "k_landmark.hpp"
#include "k_merge.hpp"
#include "k_out.hpp"
#include "k_pinv.hpp"
#include "k_pinv_mm.hpp"
#include "k_probs.hpp"

namespace nys {
namespace host {

// --------------------------------------------------------- launches ---
template <typename IO, int M, int D>
int launch_nystrom(const Plan& p, Workspace* w, const void* q, const void* k, const void* v,
                   const uint8_t* mask, const float* conv_w, int conv_k, int n_iter, int init_option, void* out,
                   hipStream_t st) {
  const float s4 = 1.0f / sqrtf(sqrtf((float)D));
  LandmarkArgs la;
  la.n = p.n;
  la.H = p.H;
  la.in = p.si;
  la.m = M;
  la.mr = p.mr;
  la.L = p.L;
  la.RS = p.RS;
  la.lpw = p.lpw;
  la.BH = p.BH;
  la.scale = s4 / (float)p.L;
  la.qt = at<float>(w, p.off_qt);
  la.kt = at<float>(w, p.off_kt);
  la.qt_hi = at<__bf16>(w, p.off_qth);
  la.qt_lo = at<__bf16>(w, p.off_qtl);
  la.kt_hi = at<__bf16>(w, p.off_kth);
  la.kt_lo = at<__bf16>(w, p.off_ktl);
  la.A = at<float>(w, p.off_A);
  la.colmax = at<float>(w, p.off_colmax);
  la.rowmax = at<float>(w, p.off_rowmax);
  la.slots = at<unsigned long long>(w, p.off_slots);
  if (!p.landmarks_ready)  // else the module's projection formed them in its epilogue
    HIP_TRY(launch("k_landmark", k_landmark<IO, M, D>, dim3(M / p.lpw, p.BH), dim3(256), 0, st, (const IO*)q,
                   (const IO*)k, la));
  // the pseudo-inverse encoding (bf16 I/O): fp16 products up to
  // PINV_F16_MAX_ITER iterations, split bf16 beyond
  const bool f16 = sizeof(IO) == 2 && n_iter <= PINV_F16_MAX_ITER;
  size_t lds_bv = (sizeof(IO) == 2 && D == HD) ? (size_t)DMA_LDS_BYTES : (size_t)KV<IO, D>::LDS_BYTES;
  lds_bv = std::max<size_t>(lds_bv, bv_fold_bytes<bv_rows<IO, M, D>(), D>());
  // the launch's LDS (B V blocks and the chosen encoding's pseudo-inverse
  // blocks), and the most either encoding needs (for the occupancy bound)
  size_t lds2 = lds_bv, lds_max = lds_bv;
  if constexpr (M <= 128) {
    const size_t pf = sizeof(IO) == 4 ? pinv_lds_bytes_f32<M>() : pinv_lds_bytes<M, true>();
    const size_t ps = sizeof(IO) == 4 ? pinv_lds_bytes_f32<M>() : pinv_lds_bytes<M, false>();
    lds2 = std::max(lds_bv, f16 ? pf : ps);
    lds_max = std::max({lds_bv, pf, ps});
  }
  // the padding-landmark and ragged-tile code only in the instance that needs it
  const bool pad = p.mr < M, edge = pad || p.n % 32 != 0;
  // The original init's one rendezvous needs every pseudo-inverse block
  // resident at once.  They are the first blocks of their launch, so they
  // are dispatched first; fuse only while they fit in half of the slots the
  // device offers the launch (and at most 128, the slots one wave polls).
  static const int fuse_cap = [&] {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    // every instance has the same block size; the largest LDS of either
    // encoding gives a bound that holds for both
    const void* kern = reinterpret_cast<const void*>(k_pinv_bv<IO, M, true, D>);
    if (allow_lds(k_pinv_bv<IO, M, true, D>, lds_max) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * bv_launch_waves<IO, M, D>(), lds_max) !=
            hipSuccess)
      return 0;
    return std::min(FUSED_GRAM_MAX_BLOCKS, per_cu * cus / 2);
  }();
  // the pseudo-inverse blocks form A themselves only at d = 64 (their LDS
  // plan holds 64-channel landmarks)
  const bool fuse_gram = D == HD && M <= 128 && (init_option != 0 || p.npinv <= fuse_cap);
  // More than 128 landmarks with bf16 I/O and 1 .. 8 iterations: the
  // expanded three-level iteration on fp16 products (k_pinv_mm.hpp), from
  // a row-split Gram.  Otherwise (float32 I/O, n_iter 0 or above 8) the
  // one-block Gram and the literal four-product iteration.  (On a side
  // stream beside the B V launch the chain was slower, 234 against 206 us
  // at 1 x 4 x 65536, m = 256: the B V blocks hold every CU, so the side
  // launches only queue behind them.)
  constexpr bool MM_OK = M > 128 && sizeof(IO) == 2;
  const bool mm_path = MM_OK && n_iter >= 1 && n_iter <= PINV_F16_MAX_ITER;
  const hipStream_t pst = st;  // stream of the pseudo-inverse launches
  // Blocks of the B V launch before its B V blocks: the pseudo-inverse
  // blocks (m <= 128), or above 128 landmarks at d = 64 the row-split Gram
  // (a launch of its own at other head sizes, whose B V launch keeps its LDS
  // plan).
  constexpr bool GRAM_IN_BV = MM_OK && D == HD;
  int npre = p.npinv;
  if constexpr (MM_OK) {
    if (mm_path) {
      constexpr int grl = gram_rows_lds_bytes<M, D>();
      if constexpr (GRAM_IN_BV) {
        npre = gram_rows_blocks<M>(p.BH);
        lds2 = std::max<size_t>(lds2, grl);
      } else {
        HIP_TRY(allow_lds(k_gram_rows<M, D>, grl));
        HIP_TRY(launch("k_gram_rows", k_gram_rows<M, D>, dim3(gram_rows_blocks<M>(p.BH)), dim3(256), (uint32_t)grl,
                       pst, la, at<float>(w, p.off_AT), at<u16>(w, p.off_T1), at<float>(w, p.off_colpart),
                       at<float>(w, p.off_rowpart)));
      }
    }
  }
  if (!fuse_gram && !mm_path) {
    constexpr size_t glds = gram_lds_bytes<M, sizeof(IO) == 4, D>();
    HIP_TRY(allow_lds(k_gram<M, sizeof(IO) == 4, D>, glds));
    HIP_TRY(launch("k_gram", k_gram<M, sizeof(IO) == 4, D>, dim3(p.BH), dim3(64 * gram_waves<M>()), (uint32_t)glds,
                   st, la));
  }

  PinvArgs pa;
  pa.A = la.A;
  pa.colmax = la.colmax;
  pa.rowmax = la.rowmax;
  pa.Z = at<float>(w, p.off_Z);
  pa.cscale = at<float>(w, p.off_cscale);
  pa.BH = p.BH;
  pa.n_iter = n_iter;
  pa.init_option = init_option;
  pa.f16 = f16 ? 1 : 0;
  pa.fuse_gram = fuse_gram ? 1 : 0;
  pa.npinv = npre;
  pa.record = p.record ? 1 : 0;
  pa.spins = g_spins;
  pa.status = at<unsigned>(w, STATUS_OFF);
  pa.la = la;
  pa.gAT = at<float>(w, p.off_AT);
  pa.gA16 = at<u16>(w, p.off_T1);
  pa.colpart = at<float>(w, p.off_colpart);
  pa.rowpart = at<float>(w, p.off_rowpart);
  BvArgs ba;
  ba.BH = p.BH;
  ba.k = k;
  ba.v = v;
  ba.key_mask = mask;
  ba.qt_hi = la.qt_hi;
  ba.qt_lo = la.qt_lo;
  ba.pmax = at<float>(w, p.off_pmax);
  ba.psum = at<float>(w, p.off_psum);
  ba.pacc = at<float>(w, p.off_pacc);
  ba.n = p.n;
  ba.H = p.H;
  ba.ntiles = p.ntiles;
  ba.lscale = s4;
  ba.in = p.si;
  constexpr int RG = bv_row_groups<IO, M, D>();
  // The plan sizes the key chunks for two resident blocks per CU beside the
  // pseudo-inverse blocks.  Where the instance that runs holds fewer (its
  // registers or LDS), or other blocks precede the B V blocks, fewer and
  // longer chunks keep the launch to one round: a second round of B V
  // blocks would start only as the first ends.  (At 1 x 8 x 16384 with 128
  // landmarks one block fits a CU: 496 B V blocks ran in two rounds.)  The
  // chunk count never grows past the plan's, which sizes the partials.
  int S = p.S, tpc = p.tpc;
  // blocks per CU of each instance (by edge and encoding) at the LDS size
  // it was last launched with
  static int occ[2][2] = {{-1, -1}, {-1, -1}}, cus = 0;
  static size_t occ_lds[2][2] = {{0, 0}, {0, 0}};
  auto launch_bv = [&](auto kern) -> int {
    HIP_TRY(allow_lds(kern, lds2));
    int& per_cu = occ[edge ? 1 : 0][f16 ? 1 : 0];
    size_t& per_lds = occ_lds[edge ? 1 : 0][f16 ? 1 : 0];
    if (per_cu < 0 || per_lds != lds2) {
      int dev = 0, pc = 0, nc = 0;
      HIP_TRY(hipGetDevice(&dev));
      HIP_TRY(hipDeviceGetAttribute(&nc, hipDeviceAttributeMultiprocessorCount, dev));
      HIP_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&pc, reinterpret_cast<const void*>(kern),
                                                           64 * bv_launch_waves<IO, M, D>(), lds2));
      cus = nc;
      per_cu = pc;
      per_lds = lds2;
    }
    const int resident = per_cu * cus;
    if (per_cu >= 1) {
      const int target = std::max(p.BH, resident - npre);
      const int s1 = std::max(1, std::min(p.ntiles, target / (p.BH * RG)));
      const int t1 = (p.ntiles + s1 - 1) / s1;
      const int s2 = (p.ntiles + t1 - 1) / t1;
      if (s2 < S) {
        S = s2;
        tpc = t1;
      }
    }
    ba.S = S;
    ba.tpc = tpc;
    const int nbv = RG == 1 ? p.BH * S : 8 * RG * ((p.BH * S + 7) / 8);
    HIP_TRY(launch("k_pinv_bv", kern, dim3(npre + nbv), dim3(64 * bv_launch_waves<IO, M, D>()), (uint32_t)lds2,
                   st, pa, ba, npre));
    return NYS_OK;
  };
  int brc;
  if constexpr (sizeof(IO) == 2 && M <= 128) {
    if (f16)
      brc = edge ? launch_bv(k_pinv_bv<IO, M, true, D, true>) : launch_bv(k_pinv_bv<IO, M, false, D, true>);
    else
      brc = edge ? launch_bv(k_pinv_bv<IO, M, true, D, false>) : launch_bv(k_pinv_bv<IO, M, false, D, false>);
  } else {
    brc = edge ? launch_bv(k_pinv_bv<IO, M, true, D>) : launch_bv(k_pinv_bv<IO, M, false, D>);
  }
  if (brc != NYS_OK) return brc;

  const float* Zfinal = pa.Z;
  if constexpr (MM_OK) {
    if (mm_path) {
      PinvMMArgs mm;
      mm.A = la.A;
      mm.AT = at<float>(w, p.off_AT);
      mm.A16 = at<u16>(w, p.off_T1);
      mm.Z = pa.Z;
      mm.Z16 = at<u16>(w, p.off_Z2);
      mm.Zt16 = at<u16>(w, p.off_Zt);
      mm.X16 = at<u16>(w, p.off_X);
      mm.Xt16 = at<u16>(w, p.off_Xt);
      mm.X2t16 = at<u16>(w, p.off_X2t);
      mm.W = at<float>(w, p.off_T2);
      mm.W16 = at<u16>(w, p.off_Zt2);
      mm.pa = pa;
      mm.colpart = at<float>(w, p.off_colpart);
      mm.colmax = la.colmax;
      mm.rowmax = la.rowmax;
      mm.rowpart = at<float>(w, p.off_rowpart);
      constexpr int NT2 = (M / PMM_T) * (M / PMM_T);
      constexpr int l1 = pinv_mm_lds_bytes<M, 1>(), l2 = pinv_mm_lds_bytes<M, 2>(), l3 = pinv_mm_lds_bytes<M, 3>();
      HIP_TRY(allow_lds(k_pinv_mm<M, 1>, l1));
      HIP_TRY(allow_lds(k_pinv_mm<M, 2>, l2));
      HIP_TRY(allow_lds(k_pinv_mm<M, 3>, l3));
      for (int it = 0; it < n_iter; ++it) {
        mm.first = it == 0 ? 1 : 0;
        HIP_TRY(launch("k_pinv_mm1", k_pinv_mm<M, 1>, dim3(pinv_mm_grid(NT2, p.BH)), dim3(256), (uint32_t)l1, pst,
                       mm));
        HIP_TRY(launch("k_pinv_mm2", k_pinv_mm<M, 2>, dim3(pinv_mm_grid(2 * NT2, p.BH)), dim3(256), (uint32_t)l2,
                       pst, mm));
        HIP_TRY(launch("k_pinv_mm3", k_pinv_mm<M, 3>, dim3(pinv_mm_grid(NT2, p.BH)), dim3(256), (uint32_t)l3, pst,
                       mm));
      }
      Zfinal = pa.Z;
    }
  }
  if constexpr (M > 128) if (!mm_path) {
    HIP_TRY(launch("k_pinv_init", k_pinv_init, dim3((M / 32) * (M / 32), p.BH), dim3(256), 0, st, pa, M));
    float* Zc = pa.Z;
    float* Zn = at<float>(w, p.off_Z2);
    float* X = at<float>(w, p.off_X);
    float* T1 = at<float>(w, p.off_T1);
    float* T2 = at<float>(w, p.off_T2);
    const dim3 gg((M / 32) * (M / 32), p.BH);
    for (int it = 0; it < n_iter; ++it) {
      HIP_TRY(launch("k_pinv_gemm", k_pinv_gemm<sizeof(IO) == 4, M>, gg, dim3(256), 0, st, (const float*)pa.A, (const float*)Zc, X,
                     0.f, 1.f));
      HIP_TRY(launch("k_pinv_gemm", k_pinv_gemm<sizeof(IO) == 4, M>, gg, dim3(256), 0, st, (const float*)X, (const float*)X, T1,
                     7.f, 1.f));
      HIP_TRY(launch("k_pinv_gemm", k_pinv_gemm<sizeof(IO) == 4, M>, gg, dim3(256), 0, st, (const float*)X, (const float*)T1, T2,
                     15.f, 1.f));
      HIP_TRY(launch("k_pinv_gemm", k_pinv_gemm<sizeof(IO) == 4, M>, gg, dim3(256), 0, st, (const float*)Zc, (const float*)T2, Zn,
                     13.f, 0.25f));
      std::swap(Zc, Zn);
    }
    Zfinal = Zc;
  }

  MergeArgs ma;
  ma.pmax = ba.pmax;
  ma.psum = ba.psum;
  ma.pacc = ba.pacc;
  ma.Z = Zfinal;
  ma.BV = at<float>(w, p.off_BV);
  ma.W = at<float>(w, p.off_W);
  ma.wf_hi = at<__bf16>(w, p.off_wfh);
  ma.wf_lo = at<__bf16>(w, p.off_wfl);
  ma.S = S;
  ma.BH = p.BH;
  ma.lse = p.bwd ? at<float>(w, p.off_lse) : nullptr;
  // threads per block: enough chunk subsets per row that each thread folds
  // one batch of 8 chunks (up to 1024 threads; 512 for m = 32)
  const int need = M * ((S + 7) / 8);
  // the bf16 output pass at d = 64 takes W^T in its own channel order
  constexpr bool B16 = sizeof(IO) == 2 && D == HD;
  constexpr int NT_MAX = M >= 64 ? 1024 : 512;
  const dim3 mwg(mw_blocks(p.BH, D));
  if (need <= 256)
    HIP_TRY(launch("k_mw", k_mw<M, B16, 256, D>, mwg, dim3(256), 0, st, ma));
  else if (need <= 512 || NT_MAX == 512)
    HIP_TRY(launch("k_mw", k_mw<M, B16, 512, D>, mwg, dim3(512), 0, st, ma));
  else
    HIP_TRY(launch("k_mw", k_mw<M, B16, NT_MAX, D>, mwg, dim3(NT_MAX), 0, st, ma));
  if (p.bwd) return NYS_OK;  // the backward pass takes it from here

  OutArgs oa;
  oa.q = q;
  oa.v = v;
  oa.q_stream = p.inputs_fresh ? 0 : 1;
  oa.zero = at<__bf16>(w, p.off_zero);
  oa.conv_w = conv_w;
  oa.conv_k = conv_k;
  oa.kt_hi = la.kt_hi;
  oa.kt_lo = la.kt_lo;
  oa.wf_hi = ma.wf_hi;
  oa.wf_lo = ma.wf_lo;
  oa.out = out;
  oa.n = p.n;
  oa.H = p.H;
  oa.lscale = s4;
  oa.in = p.si;
  oa.out_s = p.so;
  oa.mr = p.mr;
  if constexpr (sizeof(IO) == 2 && D == HD) {
    // persistent output pass: a token range of one head per workgroup, sized
    // so the grid fills the CUs at the occupancy its LDS allows in at most
    // one resident round (a second, partial round would cost a whole
    // workgroup lifetime)
    constexpr int NW = outs_waves<M>(), UNIT = outs_unit<NW>();
    constexpr size_t lds4 = OutStreamLayout<M, NW>::LDS_BYTES;
    constexpr int per_cu = std::min<int>(4, (int)(160 * 1024 / lds4));
    const int slots = 256 * per_cu;
    const int want = std::max(1, slots / p.BH);  // workgroups per head
    const int R = UNIT * ((p.n + want * UNIT - 1) / (want * UNIT));
    const int nbh = (p.n + R - 1) / R;
    u16* const junk = at<u16>(w, p.off_junk);
    auto launch_out = [&](auto kern) -> int {
      HIP_TRY(launch("k_out_stream", kern, dim3(nbh, p.BH), dim3(64 * NW), 0u, st, oa, R, junk));
      return NYS_OK;
    };
    const int orc = conv_w != nullptr ? (pad ? launch_out(k_out_stream<M, true, true, NW>)
                                             : launch_out(k_out_stream<M, true, false, NW>))
                                      : (pad ? launch_out(k_out_stream<M, false, true, NW>)
                                             : launch_out(k_out_stream<M, false, false, NW>));
    if (orc != NYS_OK) return orc;
  } else {
    using OL = OutLayout<IO, M, D>;
    auto launch_out = [&](auto kern) -> int {
      HIP_TRY(allow_lds(kern, OL::LDS_BYTES));
      HIP_TRY(launch("k_out", kern, dim3((p.n + OL::TOK - 1) / OL::TOK, p.BH), dim3(256), (uint32_t)OL::LDS_BYTES, st,
                     oa));
      return NYS_OK;
    };
    const int orc = pad ? launch_out(k_out<IO, M, true, D>) : launch_out(k_out<IO, M, false, D>);
    if (orc != NYS_OK) return orc;
  }

  if (p.probs != nullptr) {
    ProbsArgs pr{};
    pr.q = q;
    pr.kt_hi = la.kt_hi;
    pr.kt_lo = la.kt_lo;
    pr.Z = Zfinal;
    pr.probs = p.probs;
    pr.n = p.n;
    pr.H = p.H;
    pr.mr = p.mr;
    pr.ldp = p.mr;
    pr.lscale = s4;
    pr.in = p.si;
    using PL = ProbsLayout<IO, M, D>;
    pr.grp = probs_groups(p.n, p.BH, PL::NCB);
    const int ntb = (p.n + PROBS_TOK * pr.grp - 1) / (PROBS_TOK * pr.grp);
    const dim3 grid(((ntb + 7) / 8) * 8 * PL::NCB, p.BH);
    auto launch_probs = [&](auto kern) -> int {
      HIP_TRY(allow_lds(kern, PL::LDS_BYTES));
      HIP_TRY(launch("k_probs", kern, grid, dim3(256), (uint32_t)PL::LDS_BYTES, st, pr));
      return NYS_OK;
    };
    const int prc = pad ? launch_probs(k_probs<IO, M, true, D>) : launch_probs(k_probs<IO, M, false, D>);
    if (prc != NYS_OK) return prc;
  }
  return NYS_OK;
}

template <typename IO, int D>
int dispatch_m(int m, const Plan& p, Workspace* w, const void* q, const void* k, const void* v,
               const uint8_t* mask, const float* conv_w, int conv_k, int n_iter, int init_option, void* out,
               hipStream_t st) {
#define NYS_M(MM) \
  case MM:        \
    return launch_nystrom<IO, MM, D>(p, w, q, k, v, mask, conv_w, conv_k, n_iter, init_option, out, st);
  switch (m) {
    NYS_M(32)
    NYS_M(64)
    NYS_M(96)
    NYS_M(128)
    NYS_M(160)
    NYS_M(192)
    NYS_M(224)
    NYS_M(256)
    default: break;
  }
#undef NYS_M
  return fail(NYS_ERR_UNSUPPORTED, "m=%d has no kernel instance", m);
}


}  // namespace host
}  // namespace nys
