// N:M products on dense MFMA: the pipelined SpMM of spmm_q.h with every weight fragment expanded to
// dense bf16 before v_mfma_f32_16x16x32_bf16 (the "gather + dense MFMA" form of a structured-sparse
// product).  2:8 weights always take it: gfx950's structured-sparse instructions take 2:4 operands
// only.  2:4 weights take it on request (SRA_ENGINE_DENSE_MFMA), which evaluates the SMFMAC
// products against the same pipeline doing twice the MFMA work on expanded fragments (SLoPe
// paperlayer summary §2.3 runs its 2:4 products on a sparse library; §2.1 and Lemma 2.1 give 2:8
// as a further pattern).
//
//   Out[t][row] = sum_c Act[t][c] * S[row][c]  +  sum_j U[t][j] * E(row, j)     (as spmm24.hip)
//
// Tiles follow the SMFMAC planner's choices, restricted to the metadata super-stage forms
// (C % 128 == 0) plus a 128x128 four-wave tile without super-stages that may split its reduction
// for shapes that leave CUs idle.  Results agree with the SMFMAC path to fp32 summation order.
#include "spmm_q.h"

namespace {

enum XpCfg { X256x256 = 0, X256x128 = 1, X128x64 = 2, X128x128 = 3 };

struct XpPlan {
  XpCfg cfg;
  Plan p;  // splits, stages per split, tail (the 256x256 tile's last-wave split)
};

XpPlan plan_xp(int64_t R, int64_t C, int64_t T) {
  XpPlan x{X128x128, Plan{Cfg{0, 128, 128, true}, 1, (int)(C / 64)}};
  auto tiles = [&](int br, int bt) { return ((R + br - 1) / br) * ((T + bt - 1) / bt); };
  const int nC = (int)(C / 64);
  if (tiles(256, 256) >= 512) {
    x.cfg = X256x256;
    const int64_t t = tiles(256, 256);
    if (C >= 2 * R && C % 1024 == 0 && t % 256 != 0 && t % 256 <= 128) {  // as the SMFMAC plan
      x.p.splits = 2;
      x.p.tail = true;
      x.p.stages_per_split = nC / 2;
    }
  } else if (tiles(256, 128) >= 240) {
    x.cfg = X256x128;
  } else if (tiles(128, 64) >= 240 && C >= 2048) {
    x.cfg = X128x64;
  } else {
    const int64_t t = tiles(128, 128);
    if (t < 240) {
      int s = (int)((256 + t - 1) / t);
      if (s > nC / 8) s = nC / 8;  // keep >= 8 stages per split
      if (s > 1) {
        x.p.stages_per_split = (nC + s - 1) / s;
        x.p.splits = (nC + x.p.stages_per_split - 1) / x.p.stages_per_split;
      }
    }
  }
  return x;
}

bool xp_fuse_ok(const XpPlan& x, int r) {
  return r > 0 && r <= 16 && x.p.splits == 1 && sra::tuning().spmm_fuse &&
         (x.cfg == X256x128 || x.cfg == X128x64);
}

template <int NM, bool TLAY>
void launch_xp(const XpPlan& x, const uint16_t* v, const uint32_t* m, int64_t R, int64_t C,
               const uint16_t* act, int64_t T, const sra::Epilogue& ep, uint16_t* out, float* part,
               hipStream_t s) {
  const bool fuse = ep.G != nullptr;
  switch (x.cfg) {
    case X256x256:
      launch_q<4, 8, 4, 2, 3, 4, 0, false, TLAY, false, NM>(v, m, R, C, act, T, ep, out, part, x.p, s);
      break;
    case X256x128:
      if (fuse) launch_q<4, 4, 4, 2, 3, 8, 16, false, TLAY, false, NM>(v, m, R, C, act, T, ep, out, nullptr, x.p, s);
      else launch_q<4, 4, 4, 2, 4, 8, 0, false, TLAY, false, NM>(v, m, R, C, act, T, ep, out, nullptr, x.p, s);
      break;
    case X128x64:
      if (fuse) launch_q<4, 2, 2, 2, 3, 8, 16, false, TLAY, false, NM>(v, m, R, C, act, T, ep, out, nullptr, x.p, s);
      else launch_q<4, 2, 2, 2, 4, 8, 0, false, TLAY, false, NM>(v, m, R, C, act, T, ep, out, nullptr, x.p, s);
      break;
    default:
      if constexpr (TLAY)  // the streaming layout needs super-stages: 128x128, never split
        launch_q<4, 4, 2, 2, 3, 8, 0, false, true, false, NM>(v, m, R, C, act, T, ep, out, nullptr, x.p, s);
      else
        launch_q<4, 4, 2, 2, 3, 0, 0, false, false, false, NM>(v, m, R, C, act, T, ep, out, part, x.p, s);
      break;
  }
}

}  // namespace

namespace sra {

bool spmm_xp_ok(int64_t C) { return C > 0 && C % 128 == 0; }

bool spmm_xp_fuses_adapter(int64_t R, int64_t C, int64_t T, int r) {
  if (T <= 0 || R <= 0 || !spmm_xp_ok(C)) return false;
  return xp_fuse_ok(plan_xp(R, C, T), r);
}

size_t spmm_xp_ws(int64_t R, int64_t C, int64_t T) {
  if (T <= 0 || R <= 0 || !spmm_xp_ok(C)) return 0;
  const XpPlan x = plan_xp(R, C, T);
  return x.p.splits > 1 ? (size_t)x.p.splits * T * R * sizeof(float) : 0;
}

hipError_t launch_spmm_xp_bf16(int nm, bool tiled, const uint16_t* s_vals, const uint32_t* s_meta,
                               int64_t R, int64_t C, const uint16_t* act, int64_t T,
                               const Epilogue& ep, uint16_t* out, void* ws, hipStream_t s) {
  if (T == 0 || R == 0) return hipSuccess;
  if (!spmm_xp_ok(C) || !epilogue_ok(ep, R) || (nm != 24 && nm != 28) || (tiled && nm != 24))
    return hipErrorInvalidValue;
  XpPlan x = plan_xp(R, C, T);
  if (ep.G && (!xp_fuse_ok(x, ep.r) || ep.g_ld % 8 != 0)) return hipErrorInvalidValue;
  if (tiled && x.cfg == X128x128) {  // no split on the streaming layout's 128x128 tile
    x.p.splits = 1;
    x.p.stages_per_split = (int)(C / 64);
  }
  float* part = x.p.splits > 1 ? (float*)ws : nullptr;
  if (x.p.splits > 1 && !part) return hipErrorInvalidValue;
  if (nm == 28) launch_xp<28, false>(x, s_vals, s_meta, R, C, act, T, ep, out, part, s);
  else if (tiled) launch_xp<24, true>(x, s_vals, s_meta, R, C, act, T, ep, out, part, s);
  else launch_xp<24, false>(x, s_vals, s_meta, R, C, act, T, ep, out, part, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (part) finish_split(x.p, part, R, T, out, s);
  return hipGetLastError();
}

}  // namespace sra
