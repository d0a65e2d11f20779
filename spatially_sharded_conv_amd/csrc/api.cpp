// C ABI of the layer-wise, height-sharded VAE decoder: configuration, model creation
// (weight repacking), workspace planning and the band-wise decode walker.
//
// The walker runs every layer of the decoder on all bands with one kernel launch per
// layer step, on the caller's stream and without host synchronisation.  Halo rows,
// GroupNorm statistics and the global K/V pass between bands through device memory
// (the one-device form of the exchange steps in ChituDiffusion "VAEP" feature page
// and the "Static Layer-Wise VAE Decode" operator table).  The same walker runs in a
// dry mode that only sizes the workspace.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "vaep_internal.h"
#include "../../include/vaep_steps.h"

namespace vaep {

BandLayout make_layout(int nb, const int* rows, int n_img, int frames, int W, int C) {
  BandLayout L;
  std::memset(&L, 0, sizeof(L));
  L.nb = nb;
  L.n_img = n_img;
  L.frames = frames;
  L.W = W;
  L.C = C;
  long long off = 0;
  int r0 = 0;
  for (int i = 0; i < nb; ++i) {
    L.rows[i] = rows[i];
    L.row0[i] = r0;
    L.off[i] = off;
    r0 += rows[i];
    off += (long long)n_img * (rows[i] + 2) * W * C;
  }
  L.H = r0;
  return L;
}

BandLayout upsampled(const BandLayout& L, int C) {
  int rows[kMaxBands];
  for (int i = 0; i < L.nb; ++i) rows[i] = 2 * L.rows[i];
  return make_layout(L.nb, rows, L.n_img, L.frames, 2 * L.W, C);
}

BandLayout reshaped(const BandLayout& L, int C, int n_img, int frames) {
  return make_layout(L.nb, L.rows, n_img, frames, L.W, C);
}

}  // namespace vaep

using namespace vaep;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(VAEP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

struct ParamDesc {
  std::string name;
  std::vector<int64_t> shape;
};

bool is_video(const vaep_config& c) { return c.family == VAEP_FAMILY_WAN3D; }

bool stage_ups(const vaep_config& c, int i) { return i < c.n_stages - 1; }
bool stage_time_ups(const vaep_config& c, int i) {
  return is_video(c) && stage_ups(c, i) && i < c.temporal_up_stages;
}
// bf16 stages whose spatial upsample runs in sub-pixel form on the wide conv kernel
// (64-channel K steps); its operand is the stream as bf16 hi/lo parts.
bool stage_sub_up(const vaep_config& c, int i) {
  return c.dtype == VAEP_DTYPE_BF16 && stage_ups(c, i) && c.stage_channels[i] % 64 == 0 &&
         (stage_time_ups(c, i) || c.resnets_per_stage >= 1);
}
// ... where the stage's last resnet stores its output directly as those parts.  After a
// temporal upsample the stream is split by a separate pass instead.
bool stage_sub(const vaep_config& c, int i) { return stage_sub_up(c, i) && !stage_time_ups(c, i); }
// A sub-pixel upsample whose output feeds only GroupNorm/RMSNorm and a 1x1 shortcut (the
// next stage changes the channel count) stores it as hi / lo halves: the shortcut is then
// a plain bf16 conv over both halves.
bool stage_up_split(const vaep_config& c, int i) {
  return stage_sub_up(c, i) && i + 1 < c.n_stages && c.stage_channels[i + 1] != c.stage_channels[i];
}

// Canonical parameter list (names follow the decoder structure).
std::vector<ParamDesc> param_list(const vaep_config& c) {
  std::vector<ParamDesc> P;
  const bool v = is_video(c);
  auto conv = [&](const std::string& n, int co, int ci, std::vector<int64_t> k) {
    std::vector<int64_t> s = {co, ci};
    s.insert(s.end(), k.begin(), k.end());
    P.push_back({n + ".weight", s});
    P.push_back({n + ".bias", {co}});
  };
  auto lin = [&](const std::string& n, int co, int ci) {
    P.push_back({n + ".weight", {co, ci}});
    P.push_back({n + ".bias", {co}});
  };
  auto norm = [&](const std::string& n, int ch) {
    P.push_back({n + ".weight", {ch}});
    if (!v) P.push_back({n + ".bias", {ch}});
  };
  const std::vector<int64_t> k3 = v ? std::vector<int64_t>{3, 3, 3} : std::vector<int64_t>{3, 3};
  const std::vector<int64_t> k1 = v ? std::vector<int64_t>{1, 1, 1} : std::vector<int64_t>{1, 1};
  auto resnet = [&](const std::string& p, int ci, int co) {
    norm(p + ".norm1", ci);
    conv(p + ".conv1", co, ci, k3);
    norm(p + ".norm2", co);
    conv(p + ".conv2", co, co, k3);
    if (ci != co) conv(p + ".shortcut", co, ci, k1);
  };
  const int top = c.stage_channels[0];
  conv("conv_in", top, c.z_channels, k3);
  resnet("mid.res0", top, top);
  norm("mid.attn.norm", top);
  for (const char* s : {"q", "k", "v", "out"}) lin(std::string("mid.attn.") + s, top, top);
  resnet("mid.res1", top, top);
  int prev = top;
  for (int i = 0; i < c.n_stages; ++i) {
    const int co = c.stage_channels[i];
    for (int j = 0; j < c.resnets_per_stage; ++j) {
      resnet("up" + std::to_string(i) + ".res" + std::to_string(j), prev, co);
      prev = co;
    }
    if (stage_time_ups(c, i)) conv("up" + std::to_string(i) + ".time_conv", 2 * co, co, {3, 1, 1});
    if (stage_ups(c, i)) conv("up" + std::to_string(i) + ".upsample", co, co, {3, 3});
  }
  norm("norm_out", prev);
  conv("conv_out", 3, prev, k3);
  return P;
}

// Resnets per encoder down stage: one fewer than per decoder up stage (at least one).
int encoder_resnets(const vaep_config& c) { return c.resnets_per_stage > 1 ? c.resnets_per_stage - 1 : 1; }

// Canonical parameter list of the encoder of a 2-D config: conv_in (RGB -> the narrowest
// width), down stages over the reversed decoder widths (resnets, then a stride-2 3x3 conv
// in every stage but the last), the mid block, norm_out, conv_out (2 z channels: mean and
// log-variance) and a 1x1 quant_conv.
std::vector<ParamDesc> encoder_param_list(const vaep_config& c) {
  std::vector<ParamDesc> P;
  auto conv = [&](const std::string& n, int co, int ci, int k) {
    P.push_back({n + ".weight", {co, ci, k, k}});
    P.push_back({n + ".bias", {co}});
  };
  auto norm = [&](const std::string& n, int ch) {
    P.push_back({n + ".weight", {ch}});
    P.push_back({n + ".bias", {ch}});
  };
  auto resnet = [&](const std::string& p, int ci, int co) {
    norm(p + ".norm1", ci);
    conv(p + ".conv1", co, ci, 3);
    norm(p + ".norm2", co);
    conv(p + ".conv2", co, co, 3);
    if (ci != co) conv(p + ".shortcut", co, ci, 1);
  };
  const int ns = c.n_stages;
  conv("conv_in", c.stage_channels[ns - 1], 3, 3);
  int prev = c.stage_channels[ns - 1];
  for (int i = 0; i < ns; ++i) {
    const int co = c.stage_channels[ns - 1 - i];
    for (int j = 0; j < encoder_resnets(c); ++j) {
      resnet("down" + std::to_string(i) + ".res" + std::to_string(j), prev, co);
      prev = co;
    }
    if (i < ns - 1) conv("down" + std::to_string(i) + ".downsample", co, co, 3);
  }
  resnet("mid.res0", prev, prev);
  norm("mid.attn.norm", prev);
  for (const char* s : {"q", "k", "v", "out"}) {
    P.push_back({std::string("mid.attn.") + s + ".weight", {prev, prev}});
    P.push_back({std::string("mid.attn.") + s + ".bias", {prev}});
  }
  resnet("mid.res1", prev, prev);
  norm("norm_out", prev);
  conv("conv_out", 2 * c.z_channels, prev, 3);
  conv("quant_conv", 2 * c.z_channels, 2 * c.z_channels, 1);
  return P;
}

int check_config(const vaep_config* c) {
  if (!c) return fail(VAEP_ERR_INVALID_ARG, "config is NULL");
  if (c->family != VAEP_FAMILY_KL2D && c->family != VAEP_FAMILY_WAN3D)
    return fail(VAEP_ERR_UNSUPPORTED, "unknown family %d", c->family);
  if (c->dtype != VAEP_DTYPE_F32 && c->dtype != VAEP_DTYPE_BF16)
    return fail(VAEP_ERR_UNSUPPORTED, "unknown dtype %d", c->dtype);
  if (c->n_stages < 1 || c->n_stages > VAEP_MAX_STAGES)
    return fail(VAEP_ERR_INVALID_ARG, "n_stages %d outside 1..%d", c->n_stages, VAEP_MAX_STAGES);
  if (c->z_channels < 1 || c->resnets_per_stage < 1)
    return fail(VAEP_ERR_INVALID_ARG, "z_channels and resnets_per_stage must be >= 1");
  if (!(c->eps > 0.f)) return fail(VAEP_ERR_INVALID_ARG, "eps must be > 0");
  const bool bf = c->dtype == VAEP_DTYPE_BF16;
  for (int i = 0; i < c->n_stages; ++i) {
    const int ch = c->stage_channels[i];
    if (ch < 1 || ch > 1024) return fail(VAEP_ERR_INVALID_ARG, "stage_channels[%d] = %d outside 1..1024", i, ch);
    if (bf && ch % 32 != 0)
      return fail(VAEP_ERR_UNSUPPORTED, "bf16 kernels need channel counts that are multiples of 32 (stage %d: %d)", i, ch);
    if (!bf && ch % 4 != 0)
      return fail(VAEP_ERR_UNSUPPORTED, "fp32 kernels need channel counts that are multiples of 4 (stage %d: %d)", i, ch);
    if (c->family == VAEP_FAMILY_KL2D && (c->norm_groups < 1 || ch % c->norm_groups != 0))
      return fail(VAEP_ERR_INVALID_ARG, "norm_groups %d does not divide %d", c->norm_groups, ch);
  }
  if (c->family == VAEP_FAMILY_WAN3D && (c->temporal_up_stages < 0 || c->temporal_up_stages > c->n_stages - 1))
    return fail(VAEP_ERR_INVALID_ARG, "temporal_up_stages %d outside 0..%d", c->temporal_up_stages, c->n_stages - 1);
  const int top = c->stage_channels[0];
  if (bf && top != 128 && top != 256 && top != 384 && top != 512)
    return fail(VAEP_ERR_UNSUPPORTED, "bf16 attention supports 128/256/384/512 channels, got %d", top);
  return VAEP_OK;
}

// ------------------------------------------------------------------ model layout
struct ConvW {
  void* w = nullptr;
  float* b = nullptr;
  void* wsub = nullptr;   // phase-folded weights of a sub-pixel upsample conv (else NULL)
  int* sub_scale = nullptr;  // its fp8 products' MFMA scale (2 ints, launch_fold_subpixel_weight)
  // The same kernels for a decode on the transposed image (width bands): 3x3 spatial taps
  // transposed.  NULL for convs without spatial taps, which serve both orientations.
  void* wT = nullptr;
  void* wsubT = nullptr;
  int co = 0, ci = 0, co_pad = 0, ci_pad = 0, kt = 1, ks = 3;
  int rep = 1;            // 2: input channels repeated for an operand stored as hi / lo halves
  int kext = 0;           // K of a folded 1x1 conv on a second operand: its weights follow the
                          // taps' in every packed row (see ConvArgs::x2)
  int kext_ci = 0;        // that conv's true input channels (kext counts the hi / lo halves)
};
struct NormW {
  float* g = nullptr;
  float* b = nullptr;
  int c = 0;
};
struct ResW {
  NormW n1, n2;
  ConvW c1, c2, sc;
  // conv2 with the shortcut folded in (split input, bf16): K = conv2's taps, then the
  // shortcut's 2 x ci channels of the block input; bias = conv2's + the shortcut's
  ConvW c2x;
  bool has_sc = false;
  bool split_in = false;  // the block input arrives as bf16 hi / lo halves (norm1 and shortcut)
};
struct AttnW {
  NormW norm;
  ConvW qkv, out;
};
struct StageW {
  std::vector<ResW> res;
  bool time_up = false, up = false;
  bool sub_up = false;    // the upsample runs sub-pixel on a split stream
  bool sub = false;       // the last resnet writes that split stream (else a split pass does)
  bool up_split = false;  // the upsample writes its output as hi / lo halves for the next stage
  ConvW time_conv, up_conv;
};

}  // namespace

namespace {
// Event-bracketed launch records of one model (see vaep_profile_begin).
struct Profiler {
  bool on = false;
  int cap = 0;
  std::vector<hipEvent_t> ev;
  std::vector<vaep_profile_entry> rec;
};
}  // namespace

struct vaep_model {
  vaep_config cfg;
  int fold_norm = 0;   // vaep_model_set_norm_fold
  int poison_halos = 0;   // vaep_model_set_halo_poison
  void* mem = nullptr;
  size_t mem_bytes = 0;
  Profiler prof;
  ConvW conv_in;
  ResW mid0, mid1;
  AttnW attn;
  std::vector<StageW> stages;
  NormW norm_out;
  ConvW conv_out;
};

// Encoder of a 2-D config (the tiled encode): the decoder's mirror.
struct EncStageW {
  std::vector<ResW> res;
  bool down = false;   // a stride-2 3x3 conv ends the stage
  ConvW down_conv;
};

struct vaep_encoder {
  vaep_config cfg;
  void* mem = nullptr;
  size_t mem_bytes = 0;
  ConvW conv_in;
  std::vector<EncStageW> stages;
  ResW mid0, mid1;
  AttnW attn;
  NormW norm_out;
  ConvW conv_out, quant;
};

namespace {

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int round_up(int v, int a) { return (v + a - 1) / a * a; }

// Carves the model's single allocation; first pass sizes, second pass assigns.
struct Carver {
  char* base = nullptr;
  size_t used = 0;
  void* take(size_t bytes) {
    void* p = base ? base + used : nullptr;
    used = align_up(used + bytes, 256);
    return p;
  }
};

struct Builder {
  const vaep_config& c;
  const void* const* params;
  std::map<std::string, int> index;
  Carver carve;
  hipStream_t st;
  bool dry;
  int dtype;
  hipError_t err = hipSuccess;

  const void* P(const std::string& n) const { return params ? params[index.at(n)] : nullptr; }
  void ok(hipError_t e) {
    if (err == hipSuccess && e != hipSuccess) err = e;
  }

  ConvW conv(const std::string& n, int co, int ci, int kt, int ks, int co_pad_to = 0, int rep = 1) {
    ConvW w;
    const bool bf = dtype == VAEP_DTYPE_BF16;
    w.co = co;
    w.ci = ci;
    w.kt = kt;
    w.ks = ks;
    w.rep = rep;
    w.co_pad = bf ? round_up(co, kConvTileN) : co;
    if (co_pad_to) w.co_pad = co_pad_to;
    const int ci1 = bf ? round_up(ci, 32) : ci;
    w.ci_pad = ci1 * rep;
    const int taps = kt * ks * ks;
    const size_t wbytes = (size_t)w.co_pad * taps * w.ci_pad * dtype_bytes(dtype);
    w.w = carve.take(wbytes);
    if (ks == 3) w.wT = carve.take(wbytes);
    w.b = (float*)carve.take((size_t)w.co_pad * sizeof(float));
    if (!dry) {
      ok(launch_pack_weight(P(n + ".weight"), co, ci, taps, w.w, w.co_pad, ci1, dtype, st, rep));
      if (ks == 3) ok(launch_pack_weight(P(n + ".weight"), co, ci, taps, w.wT, w.co_pad, ci1, dtype, st, rep, true));
      ok(launch_to_f32(P(n + ".bias"), co, w.b, w.co_pad, dtype, st));
    }
    return w;
  }
  NormW norm(const std::string& n, int ch) {
    NormW w;
    w.c = ch;
    w.g = (float*)carve.take(ch * sizeof(float));
    w.b = (float*)carve.take(ch * sizeof(float));
    if (!dry) {
      ok(launch_to_f32(P(n + ".weight"), ch, w.g, ch, dtype, st));
      ok(launch_to_f32(is_video(c) ? nullptr : P(n + ".bias"), ch, w.b, ch, dtype, st));
    }
    return w;
  }
  ResW resnet(const std::string& p, int ci, int co, bool split_in = false) {
    ResW r;
    const int kt = is_video(c) ? 3 : 1;
    r.n1 = norm(p + ".norm1", ci);
    r.c1 = conv(p + ".conv1", co, ci, kt, 3);
    r.n2 = norm(p + ".norm2", co);
    r.c2 = conv(p + ".conv2", co, co, kt, 3);
    r.has_sc = ci != co;
    r.split_in = split_in && r.has_sc;
    if (r.has_sc) r.sc = conv(p + ".shortcut", co, ci, 1, 1, 0, r.split_in ? 2 : 1);
    if (r.split_in && dtype == VAEP_DTYPE_BF16 && r.sc.ci_pad % 64 == 0) r.c2x = folded(r.c2, r.sc);
    return r;
  }
  // conv2 with a 1x1 conv on a second operand appended to its K (packed rows side by side)
  ConvW folded(const ConvW& c2, const ConvW& sc) {
    ConvW x = c2;
    x.kext = sc.ci_pad;
    x.kext_ci = sc.ci;
    const size_t row = (size_t)c2.kt * c2.ks * c2.ks * c2.ci_pad * 2, row2 = row + (size_t)x.kext * 2;
    x.w = carve.take(c2.co_pad * row2);
    x.wT = carve.take(c2.co_pad * row2);
    x.b = (float*)carve.take((size_t)c2.co_pad * sizeof(float));
    if (!dry) {
      for (void* dst : {x.w, x.wT}) {
        const void* src = dst == x.w ? c2.w : c2.wT;
        ok(hipMemcpy2DAsync(dst, row2, src, row, row, c2.co_pad, hipMemcpyDeviceToDevice, st));
        ok(hipMemcpy2DAsync((char*)dst + row, row2, sc.w, (size_t)x.kext * 2, (size_t)x.kext * 2, c2.co_pad,
                            hipMemcpyDeviceToDevice, st));
      }
      ok(launch_add_f32(c2.b, sc.b, x.b, c2.co_pad, st));
    }
    return x;
  }
  AttnW attention(int ch) {
    AttnW a;
    a.norm = norm("mid.attn.norm", ch);
    const bool bf = dtype == VAEP_DTYPE_BF16;
    ConvW q;
    q.co = 3 * ch;
    q.ci = ch;
    q.kt = 1;
    q.ks = 1;
    q.co_pad = bf ? round_up(3 * ch, kConvTileN) : 3 * ch;
    q.ci_pad = ch;
    const size_t eb = dtype_bytes(dtype);
    q.w = carve.take((size_t)q.co_pad * ch * eb);
    q.b = (float*)carve.take((size_t)q.co_pad * sizeof(float));
    if (!dry) {
      const char* names[3] = {"mid.attn.q", "mid.attn.k", "mid.attn.v"};
      for (int i = 0; i < 3; ++i) {
        ok(launch_pack_weight(P(std::string(names[i]) + ".weight"), ch, ch, 1,
                              (char*)q.w + (size_t)i * ch * ch * eb, ch, ch, dtype, st));
        ok(launch_to_f32(P(std::string(names[i]) + ".bias"), ch, q.b + (size_t)i * ch, ch, dtype, st));
      }
    }
    a.qkv = q;
    a.out = conv("mid.attn.out", ch, ch, 1, 1);
    return a;
  }
  void build(vaep_model& m) {
    const int kt = is_video(c) ? 3 : 1;
    const int top = c.stage_channels[0];
    m.conv_in = conv("conv_in", top, c.z_channels, kt, 3);
    m.mid0 = resnet("mid.res0", top, top);
    m.attn = attention(top);
    m.mid1 = resnet("mid.res1", top, top);
    m.stages.clear();
    int prev = top;
    for (int i = 0; i < c.n_stages; ++i) {
      StageW s;
      const int co = c.stage_channels[i];
      for (int j = 0; j < c.resnets_per_stage; ++j) {
        const bool split_in = j == 0 && i > 0 && stage_up_split(c, i - 1);
        s.res.push_back(resnet("up" + std::to_string(i) + ".res" + std::to_string(j), prev, co, split_in));
        prev = co;
      }
      s.time_up = stage_time_ups(c, i);
      if (s.time_up) s.time_conv = conv("up" + std::to_string(i) + ".time_conv", 2 * co, co, 3, 1);
      s.up = stage_ups(c, i);
      if (s.up) s.up_conv = conv("up" + std::to_string(i) + ".upsample", co, co, 1, 3);
      s.sub_up = stage_sub_up(c, i);
      s.sub = stage_sub(c, i);
      s.up_split = stage_up_split(c, i);
      if (s.sub_up) {
        ConvW& u = s.up_conv;
        const size_t fbytes = (size_t)4 * u.co_pad * 4 * 2 * u.ci_pad * 2;
        u.wsub = carve.take(fbytes);
        u.wsubT = carve.take(fbytes);
        u.sub_scale = (int*)carve.take(2 * sizeof(int));
        if (!dry) {
          const std::string wn = "up" + std::to_string(i) + ".upsample.weight";
          ok(launch_fold_subpixel_weight(P(wn), co, co, u.wsub, u.co_pad, u.sub_scale, st));
          ok(launch_fold_subpixel_weight(P(wn), co, co, u.wsubT, u.co_pad, u.sub_scale, st, true));
        }
      }
      m.stages.push_back(s);
    }
    m.norm_out = norm("norm_out", prev);
    m.conv_out = conv("conv_out", 3, prev, kt, 3);
  }
  void build_encoder(vaep_encoder& e) {
    const int ns = c.n_stages;
    int prev = c.stage_channels[ns - 1];
    e.conv_in = conv("conv_in", prev, 3, 1, 3);
    e.stages.clear();
    for (int i = 0; i < ns; ++i) {
      EncStageW s;
      const int co = c.stage_channels[ns - 1 - i];
      for (int j = 0; j < encoder_resnets(c); ++j) {
        s.res.push_back(resnet("down" + std::to_string(i) + ".res" + std::to_string(j), prev, co));
        prev = co;
      }
      s.down = i < ns - 1;
      if (s.down) s.down_conv = conv("down" + std::to_string(i) + ".downsample", co, co, 1, 3);
      e.stages.push_back(s);
    }
    e.mid0 = resnet("mid.res0", prev, prev);
    e.attn = attention(prev);
    e.mid1 = resnet("mid.res1", prev, prev);
    e.norm_out = norm("norm_out", prev);
    e.conv_out = conv("conv_out", 2 * c.z_channels, prev, 1, 3);
    e.quant = conv("quant_conv", 2 * c.z_channels, 2 * c.z_channels, 1, 1);
  }
};

// ------------------------------------------------------------------ executor
enum XIn : int { kXOp = 0, kXF32 = 1, kXSplit = 2, kXNorm = 3 };

struct Exec {
  const vaep_model* m = nullptr;
  int dtype = VAEP_DTYPE_BF16;
  hipStream_t st = nullptr;
  bool dry = true;
  // workspace regions
  char* ws = nullptr;
  void* act[4] = {nullptr, nullptr, nullptr, nullptr};
  void* qb = nullptr;
  void* kb = nullptr;
  void* vb = nullptr;
  float* scratch = nullptr;
  float* ncoef = nullptr;   // (scale, shift) of a GroupNorm apply folded into the next conv
  // sizes (dry pass)
  size_t act_bytes = 0, qkv_bytes = 0, scratch_bytes = 0, ncoef_bytes = 0;
  int launches = 0;
  Profiler* prof = nullptr;
  bool recording = false;
  vaep_profile_entry pending;

  // Bracket the next launch(es) with events when profiling is on.
  void rec_begin(const vaep_profile_entry& e) {
    recording = false;
    if (dry || !prof || !prof->on || (int)prof->rec.size() >= prof->cap) return;
    const size_t i = prof->rec.size();
    if (hipEventRecord(prof->ev[2 * i], st) != hipSuccess) return;
    pending = e;
    recording = true;
  }
  void rec_end() {
    if (!recording) return;
    const size_t i = prof->rec.size();
    if (hipEventRecord(prof->ev[2 * i + 1], st) == hipSuccess) prof->rec.push_back(pending);
    recording = false;
  }
  static vaep_profile_entry entry(int step, int n_kernels) {
    vaep_profile_entry e;
    std::memset(&e, 0, sizeof(e));
    e.step = step;
    e.n_kernels = n_kernels;
    return e;
  }
  int groups = 0;      // GroupNorm groups; 0 selects channel RMSNorm
  float eps = 1e-6f;
  // Width bands: the decode runs on the transposed image (layout rows = image columns) with
  // the transposed 3x3 kernels; the latent is read and the output written transposed.
  bool transposed = false;
  // The last conv's output whose GroupNorm tile records it wrote into `scratch` (in its
  // epilogue), and their chunk width; the next norm of exactly that buffer uses them.
  const void* gn_src = nullptr;
  int gn_src_chunk = 0;
  static constexpr int kMinGnChunk = 64;   // narrowest conv pixel tile width (halo kernel, 4 x 64)
  int base_rows = 0;   // rows of the band table's own resolution (latent rows of a decode)

  size_t eb() const { return dtype_bytes(dtype); }   // operand (normalised activation) element
  void need_act(const BandLayout& L, size_t elem) { act_bytes = std::max(act_bytes, (size_t)layout_elems(L) * elem); }
  // Debug mode: the halo slots of a band buffer a layer is about to write are filled with NaN
  // first, so a slot read before the neighbour's push (or an image-edge slot read at all)
  // poisons the result.
  int poison(void* y, const BandLayout& L, int elem_bytes) {
    if (dry || !m || !m->poison_halos) return VAEP_OK;
    hipError_t e = launch_poison_halos(y, L, elem_bytes, st);
    if (e != hipSuccess) return hip_fail(e, "halo poison");
    ++launches;
    return VAEP_OK;
  }

  size_t total() const {
    return 4 * align_up(act_bytes, 256) + 3 * align_up(qkv_bytes, 256) + align_up(scratch_bytes, 256) +
           align_up(ncoef_bytes, 256);
  }
  void assign(char* base) {
    ws = base;
    size_t o = 0;
    for (int i = 0; i < 4; ++i) {
      act[i] = base + o;
      o += align_up(act_bytes, 256);
    }
    qb = base + o;
    o += align_up(qkv_bytes, 256);
    kb = base + o;
    o += align_up(qkv_bytes, 256);
    vb = base + o;
    o += align_up(qkv_bytes, 256);
    scratch = (float*)(base + o);
    o += align_up(scratch_bytes, 256);
    ncoef = (float*)(base + o);
  }

  // xk: what the input buffer holds (kXOp: a normalised activation in the operand dtype;
  // kXF32: an fp32 conv output; kXSplit: an fp32 conv output in the sub-pixel operand
  // encoding, 4 bytes per channel).  A split input with ups runs the sub-pixel form with
  // w.wsub.
  // gn_next: a GroupNorm reads the output next; the conv may then form its tile statistics.
  // split8: a kModeBandSplit output is written in the sub-pixel operand encoding (its only
  // reader is a sub-pixel upsample conv) instead of bf16 hi / lo halves.
  // x2: the second operand of a conv with a folded 1x1 part (w.kext > 0): bf16, w.kext
  // channels per pixel in Lin's band geometry.
  // down: a stride-2 conv (Lout has half Lin's rows and width).
  int conv(const ConvW& w, const void* x, const BandLayout& Lin, int xk, void* y,
           const BandLayout& Lout, int mode, const void* res, int ups, int final_frames = 1,
           bool gn_next = false, bool split8 = false, const void* x2 = nullptr, int down = 0) {
    if (w.kext > 0) need_act(reshaped(Lin, w.kext, Lin.n_img, Lin.frames), 2);
    if (mode == kModeBand || mode == kModeTimeInterleave) need_act(Lout, 4);
    if (mode == kModeBandSplit) need_act(Lout, 2);
    need_act(Lin, xk == kXOp ? eb() : ((xk == kXF32 || xk == kXNorm) ? 4 : 2));
    gn_next = gn_next && groups > 0 && dtype == VAEP_DTYPE_BF16 &&
              (mode == kModeBand || mode == kModeBandSplit);
    if (gn_next) {
      const BandLayout Lg = mode == kModeBandSplit ? reshaped(Lout, Lout.C / 2, Lout.n_img, Lout.frames) : Lout;
      scratch_bytes = std::max(scratch_bytes, gn_partials_floats(Lg, groups, 1, kMinGnChunk) * sizeof(float));
    }
    if (dry) return VAEP_OK;
    gn_src = nullptr;
    const bool sub = xk == kXSplit && ups;
    const void* wsel = sub ? (transposed ? w.wsubT : w.wsub) : (transposed && w.ks == 3 ? w.wT : w.w);
    if (!wsel) return fail(VAEP_ERR_INVALID_ARG, "internal: conv weights missing for this orientation");
    ConvArgs a;
    std::memset(&a, 0, sizeof(a));
    a.x = x;
    a.w = wsel;
    a.bias = w.b;
    a.res = res;
    a.y = y;
    a.q = qb;
    a.k = kb;
    a.vt = vb;
    a.in = Lin;
    a.out = Lout;
    a.cin = w.ci_pad;
    a.cout = w.co;
    a.cout_pad = w.co_pad;
    a.kt = w.kt;
    a.ks = w.ks;
    a.ups = ups;
    a.down = down;
    a.mode = mode;
    a.x_f32 = xk == kXF32 ? 1 : 0;
    a.x_split = xk == kXSplit ? 1 : 0;
    a.x_norm = xk == kXNorm ? ncoef : nullptr;
    a.x_norm_act = xk == kXNorm ? 1 : 0;
    a.sub = sub ? 1 : 0;
    a.sub_scale = sub ? w.sub_scale : nullptr;
    a.split8 = split8 && mode == kModeBandSplit ? 1 : 0;
    if ((w.kext > 0) != (x2 != nullptr)) return fail(VAEP_ERR_INVALID_ARG, "internal: folded conv operand mismatch");
    a.x2 = x2;
    a.cin2 = w.kext;
    a.final_frames = final_frames;
    a.out_transposed = transposed && mode == kModeFinal ? 1 : 0;
    a.gn_part = gn_next ? reinterpret_cast<double*>(scratch) : nullptr;
    a.gn_groups = gn_next ? groups : 0;
    if (Lin.C != (xk == kXSplit ? 2 : 1) * w.ci_pad)
      return fail(VAEP_ERR_INVALID_ARG, "internal: conv input has %d channels, weight %d", Lin.C, w.ci_pad);
    if (mode == kModeBand || mode == kModeTimeInterleave || mode == kModeBandSplit) {
      const int rc = poison(y, Lout, mode == kModeBandSplit ? 2 : 4);
      if (rc) return rc;
    }
    {
      vaep_profile_entry pe = entry(VAEP_STEP_CONV, 1);
      const long long m = (long long)Lin.n_img * Lin.H * Lin.W * (ups ? 4 : 1) / (down ? 4 : 1);
      const long long k = (long long)w.kt * w.ks * w.ks * w.ci + w.kext_ci;
      pe.kt = w.kt;
      pe.ks = w.ks;
      pe.cin = w.ci;
      pe.cout = w.co;
      pe.ups = ups;
      pe.mode = mode;
      pe.pixels = m;
      pe.flops = 2.0 * (double)m * w.co * (double)k;
      const double in_b = (double)Lin.n_img * Lin.H * Lin.W * (w.ci * (xk == kXOp && w.rep == 1 ? eb() : 4.0) +
                                                               (x2 ? w.kext * 2.0 : 0.0));
      const double out_elem = mode == kModeQKV ? (double)eb() : 4.0;
      pe.bytes = in_b + (double)w.co * k * eb() + (double)m * w.co * out_elem + (res ? (double)m * w.co * 4 : 0.0);
      rec_begin(pe);
    }
    hipError_t e = launch_conv(a, dtype, st);
    if (recording) pending.kernel = a.kernel_used;
    rec_end();
    if (e != hipSuccess) return hip_fail(e, "conv launch");
    ++launches;
    if (a.gn_part && a.gn_chunk > 0) {
      gn_src = y;
      gn_src_chunk = a.gn_chunk;
    }
    return VAEP_OK;
  }

  // Whether the GroupNorm + SiLU feeding conv w (Lin -> Lout, band mode) folds into the conv's
  // operand load: the model asks for it and the conv runs on the kernel that supports it.
  bool can_fold(const ConvW& w, const BandLayout& Lin, const BandLayout& Lout) const {
    if (!m || !m->fold_norm || groups <= 0 || dtype != VAEP_DTYPE_BF16 || w.kext > 0 || w.rep != 1) return false;
    ConvArgs a;
    std::memset(&a, 0, sizeof(a));
    a.in = Lin;
    a.out = Lout;
    a.cin = w.ci_pad;
    a.cout = w.co;
    a.cout_pad = w.co_pad;
    a.kt = w.kt;
    a.ks = w.ks;
    a.mode = kModeBand;
    return Lin.C == w.ci_pad && conv_norm_fold_ok(a);
  }

  // x_split: x holds bf16 hi / lo halves of the fp32 input (L describes the logical tensor)
  // stats_only: statistics and merge only, the apply's (scale, shift) into ncoef for the next
  // conv, which folds the apply into its operand load (kXNorm)
  int norm(const NormW& w, const void* x, const BandLayout& L, void* y, int act, float* merged_out = nullptr,
           bool x_split = false, bool stats_only = false) {
    need_act(L, 4);
    // reserved for every GroupNorm, folded or not: the workspace does not depend on the fold
    if (groups > 0) ncoef_bytes = std::max(ncoef_bytes, (size_t)L.n_img * L.C * 2 * sizeof(float));
    // statistics tiles never straddle a row any band table of this decode can cut at
    const int slab_rows = base_rows > 0 ? L.H / base_rows : 1;
    if (groups > 0)
      scratch_bytes = std::max(scratch_bytes, gn_partials_floats(L, groups, slab_rows) * sizeof(float));
    if (dry) return VAEP_OK;
    // statistics already formed by the conv that wrote x
    const int pre = (groups > 0 && x == gn_src) ? gn_src_chunk : 0;
    gn_src = nullptr;
    NormArgs a;
    std::memset(&a, 0, sizeof(a));
    a.pre_chunk = pre;
    a.x = x;
    a.x_split = x_split ? 1 : 0;
    a.y = y;
    a.L = L;
    a.groups = groups;
    a.eps = eps;
    a.gamma = w.g;
    a.beta = w.b;
    a.act = act;
    a.partials = reinterpret_cast<double*>(scratch);
    a.merged_out = merged_out;
    a.slab_rows = slab_rows;
    a.stats_only = stats_only ? 1 : 0;
    a.coef_out = stats_only ? ncoef : nullptr;
    const int nk = groups > 0 ? (pre ? 2 : 3) - (stats_only ? 1 : 0) : 1;
    if (!stats_only) {
      const int rc = poison(y, L, (int)eb());
      if (rc) return rc;
    }
    {
      vaep_profile_entry pe = entry(groups > 0 ? VAEP_STEP_GROUPNORM : VAEP_STEP_RMSNORM, nk);
      const double elems = (double)L.n_img * L.H * L.W * L.C;
      pe.cin = pe.cout = L.C;
      pe.pixels = (long long)L.n_img * L.H * L.W;
      // GroupNorm: statistics read (unless the producing conv formed them) + apply read
      // (fp32) + apply write; RMSNorm: one read + write
      pe.bytes = stats_only ? (pre ? 0.0 : elems * 4.0) : elems * ((groups > 0 && !pre ? 8.0 : 4.0) + (double)eb());
      rec_begin(pe);
    }
    hipError_t e = groups > 0 ? launch_groupnorm(a, dtype, st) : launch_rmsnorm(a, dtype, st);
    rec_end();
    if (e != hipSuccess) return hip_fail(e, "norm launch");
    launches += nk;
    return VAEP_OK;
  }

  // fp32 band buffer -> bf16 hi / lo halves (2C channels), halo rows included
  int split(const void* x, const BandLayout& L, void* y) {
    if (dry) return VAEP_OK;
    vaep_profile_entry pe = entry(VAEP_STEP_MOVE, 1);
    pe.cin = pe.cout = L.C;
    pe.pixels = (long long)L.n_img * L.H * L.W;
    pe.bytes = (double)layout_elems(L) * 8.0;
    rec_begin(pe);
    hipError_t e = launch_split(reinterpret_cast<const float*>(x), L, y, st);
    rec_end();
    if (e != hipSuccess) return hip_fail(e, "split launch");
    ++launches;
    return VAEP_OK;
  }

  int attention(const AttnW& w, const void* x, const BandLayout& L, void* a_buf, void* o_buf, void* y) {
    const int c = L.C;
    qkv_bytes = std::max(qkv_bytes, (size_t)L.n_img * L.H * L.W * c * eb());
    // the key-split attention's halves live in the statistics scratch, which no GroupNorm
    // holds between the QKV projection and the output projection
    if (dtype == VAEP_DTYPE_BF16)
      scratch_bytes = std::max(scratch_bytes, (size_t)attn_part_floats(L.n_img, L.H * L.W, c) * sizeof(float));
    int rc = norm(w.norm, x, L, a_buf, 0);
    if (rc) return rc;
    rc = conv(w.qkv, a_buf, L, kXOp, nullptr, L, kModeQKV, nullptr, 0);
    if (rc) return rc;
    need_act(L, eb());
    if ((rc = poison(o_buf, L, (int)eb()))) return rc;
    if (!dry) {
      AttnArgs aa;
      std::memset(&aa, 0, sizeof(aa));
      aa.q = qb;
      aa.k = kb;
      aa.vt = vb;
      aa.o = o_buf;
      aa.L = L;
      aa.c = c;
      aa.tokens = L.H * L.W;
      aa.scale = 1.0f / std::sqrt((float)c);
      aa.part = dtype == VAEP_DTYPE_BF16 ? scratch : nullptr;
      vaep_profile_entry pe = entry(VAEP_STEP_ATTENTION, 1);
      const double nq = (double)L.n_img * L.H * L.W, nk = (double)L.H * L.W;
      pe.cin = pe.cout = c;
      pe.pixels = (long long)nq;
      pe.flops = 4.0 * nq * nk * c;
      pe.bytes = 4.0 * nq * c * (double)eb();   // Q, K, V read once, O written once
      rec_begin(pe);
      hipError_t e = launch_attention(aa, dtype, st);
      rec_end();
      if (e != hipSuccess) return hip_fail(e, "attention launch");
      ++launches;
    }
    return conv(w.out, o_buf, L, kXOp, y, L, kModeBand, x, 0, 1, true);
  }
};

// Buffers other than `cur`, in a fixed order.
void others(int cur, int* o) {
  int k = 0;
  for (int i = 0; i < 4; ++i)
    if (i != cur) o[k++] = i;
}

// split_out: store the block output as bf16 hi/lo parts (layout with 2x the channels)
// for a following split-input conv, instead of fp32.
// If r.split_in, L arrives as the hi / lo layout (2 x the block's input channels).
// Whether conv2 of a resnet runs with its shortcut folded in: the folded weights exist
// (split input, bf16) and conv2 runs on the wide kernel, which alone reads a second operand.
bool shortcut_folds(const ResW& r, const BandLayout& Lh, bool split_out) {
  if (!r.c2x.w || split_out) return false;
  ConvArgs a;
  std::memset(&a, 0, sizeof(a));
  a.in = Lh;
  a.cin = r.c2x.ci_pad;
  a.cout = r.c2x.co;
  a.cout_pad = r.c2x.co_pad;
  a.kt = r.c2x.kt;
  a.ks = r.c2x.ks;
  a.mode = kModeBand;
  // the halo kernel takes the second operand in 32-channel steps (its launch checks the
  // buffer-resource sizes)
  a.x2 = r.c2x.w;   // any non-null pointer: only the fit is asked here
  a.cin2 = r.c2x.kext;
  if (conv_halo_fits(a)) return true;
  a.x2 = nullptr;
  a.cin2 = 0;
  if (!conv_wide_fits(a)) return false;
  // the second operand's rows one tile reads stay within a buffer resource (2 GiB)
  const int bn = wide_tile(a).bn;
  for (int b = 0; b < Lh.nb; ++b)
    if ((tile_read_slots(Lh, b, a.kt, bn, false) * Lh.W + 2LL * bn) * r.c2x.kext * 2 >= (1LL << 31) - 4096)
      return false;
  return true;
}

int resnet(Exec& E, const ResW& r, int& cur, BandLayout& L, bool split_out = false) {
  int o[3];
  others(cur, o);
  const BandLayout Lx = r.split_in ? reshaped(L, L.C / 2, L.n_img, L.frames) : L;
  const BandLayout Lh = reshaped(L, r.c1.co, L.n_img, L.frames);
  const BandLayout Ly = split_out ? reshaped(L, 2 * r.c1.co, L.n_img, L.frames) : Lh;
  int rc;
  // GroupNorm + SiLU -> conv1: the apply folded into conv1's operand load where the model
  // asks for it and conv1 runs on the kernel that supports it, else a separate pass
  if (!r.split_in && E.can_fold(r.c1, Lx, Lh)) {
    if ((rc = E.norm(r.n1, E.act[cur], Lx, nullptr, 1, nullptr, false, true))) return rc;
    if ((rc = E.conv(r.c1, E.act[cur], Lx, kXNorm, E.act[o[1]], Lh, kModeBand, nullptr, 0, 1, true))) return rc;
  } else {
    if ((rc = E.norm(r.n1, E.act[cur], Lx, E.act[o[0]], 1, nullptr, r.split_in))) return rc;
    if ((rc = E.conv(r.c1, E.act[o[0]], Lx, kXOp, E.act[o[1]], Lh, kModeBand, nullptr, 0, 1, true))) return rc;
  }
  if (!shortcut_folds(r, Lh, split_out) && !split_out && E.can_fold(r.c2, Lh, Ly)) {
    // conv2 reads conv1's raw output and writes the free operand buffer; the merge first,
    // while conv1's statistics records are the latest in the scratch
    if ((rc = E.norm(r.n2, E.act[o[1]], Lh, nullptr, 1, nullptr, false, true))) return rc;
    const void* res = E.act[cur];
    if (r.has_sc) {
      if ((rc = E.conv(r.sc, E.act[cur], L, r.split_in ? kXOp : kXF32, E.act[o[2]], Lh, kModeBand, nullptr, 0)))
        return rc;
      res = E.act[o[2]];
    }
    if ((rc = E.conv(r.c2, E.act[o[1]], Lh, kXNorm, E.act[o[0]], Ly, kModeBand, res, 0, 1, true))) return rc;
    cur = o[0];
    L = Ly;
    return VAEP_OK;
  }
  if ((rc = E.norm(r.n2, E.act[o[1]], Lh, E.act[o[0]], 1))) return rc;
  if (shortcut_folds(r, Lh, split_out)) {
    // conv2 + shortcut in one conv: K runs over conv2's taps, then the block input's
    // hi / lo channels at the pixel itself; no residual pass
    if ((rc = E.conv(r.c2x, E.act[o[0]], Lh, kXOp, E.act[o[1]], Ly, kModeBand, nullptr, 0, 1, true, false,
                     E.act[cur])))
      return rc;
    cur = o[1];
    L = Ly;
    return VAEP_OK;
  }
  const void* res = E.act[cur];
  if (r.has_sc) {
    // a split input is a bf16 operand over both halves (weights repeated)
    if ((rc = E.conv(r.sc, E.act[cur], L, r.split_in ? kXOp : kXF32, E.act[o[2]], Lh, kModeBand, nullptr, 0)))
      return rc;
    res = E.act[o[2]];
  }
  // every resnet output but a split one (read by the upsample conv) feeds a norm next
  if ((rc = E.conv(r.c2, E.act[o[0]], Lh, kXOp, E.act[o[1]], Ly, split_out ? kModeBandSplit : kModeBand, res, 0, 1,
                   !split_out, split_out)))
    return rc;
  cur = o[1];
  L = Ly;
  return VAEP_OK;
}

// Decode a latent on the given bands (rows per band at latent resolution).
int walk(Exec& E, const void* latent, int B, int T, int W, const int* rows, int nb, void* out) {
  const vaep_model& m = *E.m;
  const vaep_config& c = m.cfg;
  const bool video = is_video(c);
  E.groups = video ? 0 : c.norm_groups;
  E.eps = c.eps;
  int H = 0;
  for (int i = 0; i < nb; ++i) H += rows[i];
  E.base_rows = H;
  BandLayout L = make_layout(nb, rows, B * T, T, W, m.conv_in.ci_pad);
  int rc;
  int cur = 0;
  E.need_act(L, E.eb());
  if (!E.dry) {
    hipError_t e = launch_pack(latent, c.z_channels, E.act[0], L, E.dtype, E.st, E.transposed);
    if (e != hipSuccess) return hip_fail(e, "latent pack");
    ++E.launches;
  }
  BandLayout L1 = reshaped(L, m.conv_in.co, L.n_img, T);
  if ((rc = E.conv(m.conv_in, E.act[0], L, kXOp, E.act[1], L1, kModeBand, nullptr, 0, 1, true))) return rc;
  cur = 1;
  L = L1;
  if ((rc = resnet(E, m.mid0, cur, L))) return rc;
  {
    int o[3];
    others(cur, o);
    if ((rc = E.attention(m.attn, E.act[cur], L, E.act[o[0]], E.act[o[1]], E.act[o[2]]))) return rc;
    cur = o[2];
  }
  if ((rc = resnet(E, m.mid1, cur, L))) return rc;
  for (const StageW& s : m.stages) {
    for (size_t j = 0; j < s.res.size(); ++j)
      if ((rc = resnet(E, s.res[j], cur, L, s.sub && j + 1 == s.res.size()))) return rc;
    if (s.time_up) {
      int o[3];
      others(cur, o);
      const int Tn = 2 * L.frames - 1;
      const BandLayout Lt = reshaped(L, L.C, (L.n_img / L.frames) * Tn, Tn);
      if ((rc = E.conv(s.time_conv, E.act[cur], L, kXF32, E.act[o[0]], Lt, kModeTimeInterleave, nullptr, 0))) return rc;
      if (!E.dry) {
        hipError_t e = launch_copy_frame0(E.act[cur], L, E.act[o[0]], Lt, VAEP_DTYPE_F32, E.st);
        if (e != hipSuccess) return hip_fail(e, "frame copy");
        ++E.launches;
      }
      cur = o[0];
      L = Lt;
    }
    if (s.up) {
      int o[3];
      others(cur, o);
      const BandLayout Lu = upsampled(L, (s.up_split ? 2 : 1) * s.up_conv.co);
      int src = cur;
      BandLayout Ls = L;
      if (s.sub_up && !s.sub) {   // split the fp32 stream (halo rows included) for the sub-pixel conv
        Ls = reshaped(L, 2 * L.C, L.n_img, L.frames);
        E.need_act(Ls, 2);
        src = o[1];
        if ((rc = E.split(E.act[cur], L, E.act[src]))) return rc;
      }
      if ((rc = E.conv(s.up_conv, E.act[src], Ls, s.sub_up ? kXSplit : kXF32, E.act[o[0]], Lu,
                       s.up_split ? kModeBandSplit : kModeBand, nullptr, 1, 1, true)))
        return rc;
      cur = o[0];
      L = Lu;
    }
  }
  int o[3];
  others(cur, o);
  if ((rc = E.norm(m.norm_out, E.act[cur], L, E.act[o[0]], 1))) return rc;
  (void)video;
  return E.conv(m.conv_out, E.act[o[0]], L, kXOp, out, L, kModeFinal, nullptr, 0, L.frames);
}

// Rows of nb bands that split H as evenly as possible (used to size workspaces).
std::vector<int> even_rows(int H, int nb) {
  std::vector<int> r(nb, H / nb);
  for (int i = 0; i < H % nb; ++i) r[i] += 1;
  return r;
}

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(VAEP_ERR_NOT_READY, "no HIP device: %s", hipGetErrorString(e));
  hipDeviceProp_t p;
  e = hipGetDeviceProperties(&p, dev);
  if (e != hipSuccess) return fail(VAEP_ERR_NOT_READY, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (std::strncmp(p.gcnArchName, "gfx950", 6) != 0)
    return fail(VAEP_ERR_NOT_READY, "device %d is %s; this library is built for gfx950", dev, p.gcnArchName);
  return VAEP_OK;
}

int check_latent_dims(const vaep_model* m, int batch, int frames, int h, int w) {
  if (!m) return fail(VAEP_ERR_INVALID_ARG, "model is NULL");
  if (batch < 1 || h < 1 || w < 1 || frames < 1)
    return fail(VAEP_ERR_INVALID_ARG, "latent dims must be >= 1 (batch %d frames %d h %d w %d)", batch, frames, h, w);
  if (!is_video(m->cfg) && frames != 1) return fail(VAEP_ERR_INVALID_ARG, "2-D decoder needs frames = 1");
  const long long up = 1LL << (m->cfg.n_stages - 1);
  if ((long long)h * up > (1 << 20) || (long long)w * up > (1 << 20))
    return fail(VAEP_ERR_INVALID_ARG, "latent %dx%d too large", h, w);
  return VAEP_OK;
}

// Workspace of a decode whose nb bands cut an axis of length `cut` (the other axis `other`).
int plan_bytes(const vaep_model* m, int batch, int frames, int cut, int other, int nb, bool transposed,
               size_t* bytes) {
  Exec E;
  E.m = m;
  E.dtype = m->cfg.dtype;
  E.dry = true;
  E.transposed = transposed;
  std::vector<int> rows = even_rows(cut, nb);
  int rc = walk(E, nullptr, batch, frames, other, rows.data(), nb, nullptr);
  if (rc) return rc;
  *bytes = E.total();
  return VAEP_OK;
}

// Dry pass (sizing), workspace check and the decode itself on `rows` bands of the cut axis.
int run_decode(vaep_model* model, const void* latent, int batch, int frames, int other, bool transposed,
               const std::vector<int>& rows, int axis_code, int status, void* out, void* ws, size_t ws_bytes,
               void* stream, vaep_decode_info* info) {
  const int nb = (int)rows.size();
  Exec E;
  E.m = model;
  E.dtype = model->cfg.dtype;
  E.st = (hipStream_t)stream;
  E.dry = true;
  E.transposed = transposed;
  E.prof = &model->prof;
  int rc;
  if ((rc = walk(E, latent, batch, frames, other, rows.data(), nb, out))) return rc;
  const size_t need = E.total();
  if (!ws || ws_bytes < need)
    return fail(VAEP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
  E.assign((char*)ws);
  E.dry = false;
  if ((rc = walk(E, latent, batch, frames, other, rows.data(), nb, out))) return rc;
  if (info) {
    info->bands_used = nb;
    info->fell_back = status == VAEP_WARN_FELL_BACK || axis_code == VAEP_AXIS_DENSE;
    info->n_launches = E.launches;
    info->axis = axis_code;
    info->workspace_bytes = need;
  }
  return VAEP_OK;
}

// Row counts of a validated band table along an axis of length `len`.
int table_rows(const int32_t* starts, int n, int len, const char* what, std::vector<int>& rows) {
  if (starts[0] != 0 || starts[n] != len)
    return fail(VAEP_ERR_INVALID_ARG, "%s bands must cover 0..%d (got %d..%d)", what, len, starts[0], starts[n]);
  rows.clear();
  for (int i = 0; i < n; ++i) {
    if (starts[i + 1] <= starts[i])
      return fail(VAEP_ERR_INVALID_ARG, "%s band %d is empty or reversed (%d..%d)", what, i, starts[i], starts[i + 1]);
    rows.push_back(starts[i + 1] - starts[i]);
  }
  return VAEP_OK;
}

// Clipped edge tiles of a tile grid grouped by their size (latent rows x columns), in
// raster order of first appearance: each group runs as one batch of images.
struct EdgeGroup {
  int th = 0, tw = 0;
  std::vector<int> tiles;   // gi * nc + gj
};
std::vector<EdgeGroup> edge_groups(int nr, int nc, int full_r, int full_c, int tile, int stride, int h, int w) {
  std::vector<EdgeGroup> g;
  for (int gi = 0; gi < nr; ++gi)
    for (int gj = 0; gj < nc; ++gj) {
      if (gi < full_r && gj < full_c) continue;
      const int th = std::min(tile, h - gi * stride), tw = std::min(tile, w - gj * stride);
      size_t k = 0;
      while (k < g.size() && (g[k].th != th || g[k].tw != tw)) ++k;
      if (k == g.size()) {
        g.push_back(EdgeGroup());
        g[k].th = th;
        g[k].tw = tw;
      }
      g[k].tiles.push_back(gi * nc + gj);
    }
  return g;
}

// The same bands after a stride-2 conv: rows and width halve (every band's row count even).
BandLayout halved(const BandLayout& L, int C) {
  int rows[kMaxBands];
  for (int i = 0; i < L.nb; ++i) rows[i] = L.rows[i] / 2;
  return make_layout(L.nb, rows, L.n_img, L.frames, L.W / 2, C);
}

// Encoder forward of `batch` images of H x W (multiples of 2^(n_stages-1)) as one band:
// image (NCHW, the config's dtype) -> moments (NCHW fp32, 2 z channels).
int walk_encoder(Exec& E, const vaep_encoder& e, const void* image, int B, int H, int W, void* out) {
  const vaep_config& c = e.cfg;
  E.groups = c.norm_groups;
  E.eps = c.eps;
  E.base_rows = H >> (c.n_stages - 1);   // GroupNorm statistics tiles of whole latent-row slabs
  const int rows[1] = {H};
  BandLayout L = make_layout(1, rows, B, 1, W, e.conv_in.ci_pad);
  int rc;
  E.need_act(L, E.eb());
  if (!E.dry) {
    hipError_t err = launch_pack(image, 3, E.act[0], L, E.dtype, E.st, false);
    if (err != hipSuccess) return hip_fail(err, "image pack");
    ++E.launches;
  }
  BandLayout L1 = reshaped(L, e.conv_in.co, B, 1);
  if ((rc = E.conv(e.conv_in, E.act[0], L, kXOp, E.act[1], L1, kModeBand, nullptr, 0, 1, true))) return rc;
  int cur = 1;
  L = L1;
  for (const EncStageW& st : e.stages) {
    for (const ResW& r : st.res)
      if ((rc = resnet(E, r, cur, L))) return rc;
    if (st.down) {
      int o[3];
      others(cur, o);
      const BandLayout Ld = halved(L, st.down_conv.co);
      if ((rc = E.conv(st.down_conv, E.act[cur], L, kXF32, E.act[o[0]], Ld, kModeBand, nullptr, 0, 1, false, false,
                       nullptr, 1)))
        return rc;
      cur = o[0];
      L = Ld;
    }
  }
  if ((rc = resnet(E, e.mid0, cur, L))) return rc;
  {
    int o[3];
    others(cur, o);
    if ((rc = E.attention(e.attn, E.act[cur], L, E.act[o[0]], E.act[o[1]], E.act[o[2]]))) return rc;
    cur = o[2];
  }
  if ((rc = resnet(E, e.mid1, cur, L))) return rc;
  int o[3];
  others(cur, o);
  if ((rc = E.norm(e.norm_out, E.act[cur], L, E.act[o[0]], 1))) return rc;
  const BandLayout Lz = reshaped(L, e.conv_out.co, B, 1);
  if ((rc = E.conv(e.conv_out, E.act[o[0]], L, kXOp, E.act[o[1]], Lz, kModeBand, nullptr, 0))) return rc;
  if ((rc = E.conv(e.quant, E.act[o[1]], Lz, kXF32, E.act[o[2]], Lz, kModeBand, nullptr, 0))) return rc;
  if (!E.dry) {
    hipError_t err = launch_unpack(E.act[o[2]], Lz, out, e.quant.co, VAEP_DTYPE_F32, E.st);
    if (err != hipSuccess) return hip_fail(err, "moments gather");
    ++E.launches;
  }
  return VAEP_OK;
}

// Workspace of one whole-image encode of `batch` images of H x W.
int encode_plan_bytes(const vaep_encoder* e, int batch, int H, int W, size_t* bytes) {
  Exec E;
  E.dtype = e->cfg.dtype;
  E.dry = true;
  int rc = walk_encoder(E, *e, nullptr, batch, H, W, nullptr);
  if (rc) return rc;
  *bytes = E.total();
  return VAEP_OK;
}

// Dry pass (sizing), workspace check and the encode of `batch` images of H x W.
int run_encode(const vaep_encoder* e, const void* image, int batch, int H, int W, void* out, void* ws,
               size_t ws_bytes, void* stream, int* launches) {
  Exec E;
  E.dtype = e->cfg.dtype;
  E.st = (hipStream_t)stream;
  E.dry = true;
  int rc;
  if ((rc = walk_encoder(E, *e, image, batch, H, W, out))) return rc;
  const size_t need = E.total();
  if (!ws || ws_bytes < need)
    return fail(VAEP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
  E.assign((char*)ws);
  E.dry = false;
  if ((rc = walk_encoder(E, *e, image, batch, H, W, out))) return rc;
  if (launches) *launches += E.launches;
  return VAEP_OK;
}

// Tiled encode: tiles of tile x tile latent pixels (tile * up image pixels) every stride.
struct EncTilePlan {
  int up = 1, lh = 0, lw = 0;
  int nr = 0, nc = 0, nfull = 0, full_r = 0, full_c = 0;
  long long planes = 0;      // moment planes: batch * 2 z
  long long slot_elems = 0;  // fp32 elements of one tile slot (largest tile)
  std::vector<EdgeGroup> edges;
  size_t enc_bytes = 0, img_bytes = 0, stage_bytes = 0, store_bytes = 0, total = 0;
};

int enc_tile_plan(const vaep_encoder* e, int batch, int H, int W, int tile, int stride, EncTilePlan* tp) {
  if (tile < 1 || stride < 1 || stride > tile)
    return fail(VAEP_ERR_INVALID_ARG, "tile %d and stride %d must satisfy 1 <= stride <= tile", tile, stride);
  tp->up = 1 << (e->cfg.n_stages - 1);
  tp->lh = H / tp->up;
  tp->lw = W / tp->up;
  tp->nr = (tp->lh + stride - 1) / stride;
  tp->nc = (tp->lw + stride - 1) / stride;
  tp->planes = (long long)batch * 2 * e->cfg.z_channels;
  const int th = std::min(tile, tp->lh), tw = std::min(tile, tp->lw);
  tp->slot_elems = tp->planes * th * tw;
  int full_r = 0, full_c = 0;
  for (int i = 0; i < tp->lh; i += stride) full_r += i + tile <= tp->lh ? 1 : 0;
  for (int j = 0; j < tp->lw; j += stride) full_c += j + tile <= tp->lw ? 1 : 0;
  tp->full_r = full_r;
  tp->full_c = full_c;
  tp->nfull = full_r * full_c;
  // the full tiles, then each edge group, run as one batch each in the same workspace; the
  // edge groups' moments pass through a staging area on their way to the slots
  tp->edges = edge_groups(tp->nr, tp->nc, full_r, full_c, tile, stride, tp->lh, tp->lw);
  const size_t img_px = (size_t)batch * 3 * dtype_bytes(e->cfg.dtype) * tp->up * tp->up;
  size_t enc = 0, img = 0, stage = 0;
  int rc;
  if (tp->nfull > 0) {
    if ((rc = encode_plan_bytes(e, batch * tp->nfull, tile * tp->up, tile * tp->up, &enc))) return rc;
    img = (size_t)tp->nfull * tile * tile * img_px;
  }
  for (const EdgeGroup& g : tp->edges) {
    const int n = (int)g.tiles.size();
    size_t b = 0;
    if ((rc = encode_plan_bytes(e, batch * n, g.th * tp->up, g.tw * tp->up, &b))) return rc;
    enc = std::max(enc, b);
    img = std::max(img, (size_t)n * g.th * g.tw * img_px);
    stage = std::max(stage, (size_t)n * (size_t)tp->planes * g.th * g.tw * sizeof(float));
  }
  tp->enc_bytes = align_up(enc, 256);
  tp->img_bytes = align_up(img, 256);
  tp->stage_bytes = align_up(stage, 256);
  tp->store_bytes = (size_t)tp->nr * tp->nc * tp->slot_elems * sizeof(float);
  tp->total = tp->enc_bytes + tp->img_bytes + tp->stage_bytes + tp->store_bytes;
  return VAEP_OK;
}

int check_image_dims(const vaep_encoder* e, int batch, int H, int W) {
  if (!e) return fail(VAEP_ERR_INVALID_ARG, "encoder is NULL");
  const int up = 1 << (e->cfg.n_stages - 1);
  if (batch < 1 || H < up || W < up || H % up != 0 || W % up != 0)
    return fail(VAEP_ERR_INVALID_ARG, "image %dx%d (batch %d) must be positive multiples of %d", H, W, batch, up);
  if ((long long)H * W > (1LL << 26)) return fail(VAEP_ERR_INVALID_ARG, "image %dx%d too large", H, W);
  return VAEP_OK;
}

// Tiled decode (overlap-blending baseline): tile grid, workspace carve-up.
struct TilePlan {
  int nr = 0, nc = 0;          // tile rows and columns
  int nfull = 0;               // tiles of the full tile size (decoded together as one batch)
  int full_r = 0, full_c = 0;  // ... the first full_r tile rows x full_c tile columns
  int up = 1;                  // output pixels per latent pixel
  int blend = 0;               // overlap in output rows / columns
  long long planes = 0;        // output planes: batch * 3 * output frames
  long long slot_elems = 0;    // fp32 elements of one tile slot (largest tile)
  std::vector<EdgeGroup> edges;
  size_t dec_bytes = 0, lat_bytes = 0, stage_bytes = 0, store_bytes = 0, total = 0;
};

int tile_plan(const vaep_model* m, int batch, int frames, int h, int w, int tile, int stride, TilePlan* tp) {
  if (tile < 1 || stride < 1 || stride > tile)
    return fail(VAEP_ERR_INVALID_ARG, "tile %d and stride %d must satisfy 1 <= stride <= tile", tile, stride);
  tp->nr = (h + stride - 1) / stride;
  tp->nc = (w + stride - 1) / stride;
  tp->up = 1 << (m->cfg.n_stages - 1);
  tp->blend = (tile - stride) * tp->up;
  int t_out = frames;
  for (int i = 0; i < m->cfg.n_stages; ++i)
    if (stage_time_ups(m->cfg, i)) t_out = 2 * t_out - 1;
  tp->planes = (long long)batch * 3 * t_out;
  const int th = std::min(tile, h), tw = std::min(tile, w);
  tp->slot_elems = tp->planes * (long long)th * tp->up * tw * tp->up;
  // tiles lying wholly inside the image share one size and decode as one batch; the
  // clipped edge tiles decode as one batch per tile size
  int full_r = 0, full_c = 0;
  for (int i = 0; i < h; i += stride) full_r += i + tile <= h ? 1 : 0;
  for (int j = 0; j < w; j += stride) full_c += j + tile <= w ? 1 : 0;
  tp->full_r = full_r;
  tp->full_c = full_c;
  tp->nfull = full_r * full_c;
  // every batch (the full tiles, then each edge group) decodes in the same workspace; the
  // edge groups' outputs pass through a staging area on their way to the slots
  tp->edges = edge_groups(tp->nr, tp->nc, full_r, full_c, tile, stride, h, w);
  const size_t lat_px = (size_t)batch * m->cfg.z_channels * frames * dtype_bytes(m->cfg.dtype);
  size_t dec = 0, lat = 0, stage = 0;
  int rc;
  if (tp->nfull > 0) {
    if ((rc = plan_bytes(m, batch * tp->nfull, frames, tile, tile, 1, false, &dec))) return rc;
    lat = (size_t)tp->nfull * tile * tile * lat_px;
  }
  for (const EdgeGroup& g : tp->edges) {
    const int n = (int)g.tiles.size();
    size_t b = 0;
    if ((rc = plan_bytes(m, batch * n, frames, g.th, g.tw, 1, false, &b))) return rc;
    dec = std::max(dec, b);
    lat = std::max(lat, (size_t)n * g.th * g.tw * lat_px);
    stage = std::max(stage, (size_t)n * (size_t)tp->planes * g.th * tp->up * g.tw * tp->up * sizeof(float));
  }
  tp->dec_bytes = align_up(dec, 256);
  tp->lat_bytes = align_up(lat, 256);
  tp->stage_bytes = align_up(stage, 256);
  tp->store_bytes = (size_t)tp->nr * tp->nc * tp->slot_elems * sizeof(float);
  tp->total = tp->dec_bytes + tp->lat_bytes + tp->stage_bytes + tp->store_bytes;
  return VAEP_OK;
}

// The per-request axis policy: the longer axis that gives every shard at least one latent
// row (the kernel radius at latent resolution), width on ties; the tile decode when neither
// axis covers the shards; one dense band for a single shard.
int select_axis(int h, int w, int n) {
  if (n <= 1) return VAEP_AXIS_DENSE;
  const bool cover_h = h >= n, cover_w = w >= n;
  if (cover_w && (w >= h || !cover_h)) return VAEP_AXIS_WIDTH;
  if (cover_h) return VAEP_AXIS_HEIGHT;
  return VAEP_AXIS_TILE;
}

// Tile geometry of the tile strategy: latent tiles of 32 rows and columns every 24 (the
// strategy page names the tile attributes but not their values).
constexpr int kShardTile = 32, kShardTileStride = 24;


// ------------------------------------------------------------------ step helpers
int step_bands(const int32_t* rs, int nb, int h, std::vector<int>& rows) {
  if (!rs) return fail(VAEP_ERR_INVALID_ARG, "row_starts is NULL");
  if (nb < 1 || nb > kMaxBands) return fail(VAEP_ERR_INVALID_ARG, "n_bands %d outside 1..%d", nb, kMaxBands);
  if (rs[0] != 0 || rs[nb] != h) return fail(VAEP_ERR_INVALID_ARG, "bands must cover rows 0..%d", h);
  rows.clear();
  for (int i = 0; i < nb; ++i) {
    if (rs[i + 1] <= rs[i]) return fail(VAEP_ERR_INVALID_ARG, "band %d is empty or reversed", i);
    rows.push_back(rs[i + 1] - rs[i]);
  }
  return VAEP_OK;
}

int step_dims(int dtype, int batch, int frames, int c, int h, int w) {
  if (dtype != VAEP_DTYPE_F32 && dtype != VAEP_DTYPE_BF16) return fail(VAEP_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (batch < 1 || frames < 1 || c < 1 || h < 1 || w < 1)
    return fail(VAEP_ERR_INVALID_ARG, "dims must be >= 1 (batch %d frames %d c %d h %d w %d)", batch, frames, c, h, w);
  return VAEP_OK;
}

// Sizes the step workspace on the first pass (base == NULL) and hands out pointers on the second.
int step_finish_sizing(const Carver& cv, void* ws, size_t ws_bytes, size_t* bytes_out, bool* sized) {
  *sized = false;
  if (!ws) {
    if (!bytes_out) return fail(VAEP_ERR_INVALID_ARG, "ws and bytes_out are both NULL");
    *bytes_out = cv.used;
    *sized = true;
    return VAEP_OK;
  }
  if (ws_bytes < cv.used) return fail(VAEP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", cv.used, ws_bytes);
  return VAEP_OK;
}

int norm_channels_ok(int dtype, int c) {
  (void)dtype;   // norm inputs are fp32 conv outputs: 4 channels per 16-byte load, 256 threads
  if (c % 4 != 0 || c > 1024) return fail(VAEP_ERR_UNSUPPORTED, "norm kernels need channels %% 4 == 0 and <= 1024");
  return VAEP_OK;
}

}  // namespace

namespace vaep {
int set_error(int code, const char* msg) { return fail(code, "%s", msg); }
}  // namespace vaep

extern "C" {

const char* vaep_last_error(void) { return g_err.c_str(); }

const char* vaep_version(void) { return "vaep 0.1 gfx950"; }

int vaep_config_preset(int id, vaep_config* out) {
  if (!out) return fail(VAEP_ERR_INVALID_ARG, "out is NULL");
  vaep_config c;
  std::memset(&c, 0, sizeof(c));
  c.eps = 1e-6f;
  if (id == 1) {
    c.family = VAEP_FAMILY_KL2D;
    c.dtype = VAEP_DTYPE_F32;
    c.z_channels = 4;
    c.n_stages = 2;
    c.stage_channels[0] = 64;
    c.stage_channels[1] = 32;
    c.resnets_per_stage = 2;
    c.norm_groups = 8;
  } else if (id >= 2 && id <= 4) {
    c.family = VAEP_FAMILY_KL2D;
    c.dtype = VAEP_DTYPE_BF16;
    c.z_channels = 16;
    c.n_stages = 4;
    const int ch[4] = {512, 512, 256, 128};
    for (int i = 0; i < 4; ++i) c.stage_channels[i] = ch[i];
    c.resnets_per_stage = 3;
    c.norm_groups = 32;
  } else if (id == 5) {
    c.family = VAEP_FAMILY_WAN3D;
    c.dtype = VAEP_DTYPE_BF16;
    c.z_channels = 16;
    c.n_stages = 4;
    const int ch[4] = {384, 384, 192, 96};
    for (int i = 0; i < 4; ++i) c.stage_channels[i] = ch[i];
    c.resnets_per_stage = 2;
    c.norm_groups = 0;
    c.temporal_up_stages = 2;
  } else {
    return fail(VAEP_ERR_INVALID_ARG, "unknown preset %d (1..5)", id);
  }
  *out = c;
  return VAEP_OK;
}

int vaep_param_count(const vaep_config* cfg) {
  int rc = check_config(cfg);
  if (rc) return rc;
  return (int)param_list(*cfg).size();
}

int vaep_param_info(const vaep_config* cfg, int j, char* name, int name_cap, int64_t shape[5], int* ndim) {
  int rc = check_config(cfg);
  if (rc) return rc;
  const auto P = param_list(*cfg);
  if (j < 0 || j >= (int)P.size()) return fail(VAEP_ERR_INVALID_ARG, "parameter index %d outside 0..%d", j, (int)P.size() - 1);
  if (name && name_cap > 0) {
    std::strncpy(name, P[j].name.c_str(), name_cap - 1);
    name[name_cap - 1] = 0;
  }
  if (shape)
    for (size_t i = 0; i < P[j].shape.size() && i < 5; ++i) shape[i] = P[j].shape[i];
  if (ndim) *ndim = (int)P[j].shape.size();
  return VAEP_OK;
}

int vaep_model_create(const vaep_config* cfg, const void* const* params, int n_params, void* stream,
                      vaep_model** out) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!out) return fail(VAEP_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  const auto P = param_list(*cfg);
  if (!params) return fail(VAEP_ERR_INVALID_ARG, "params is NULL");
  if (n_params != (int)P.size()) return fail(VAEP_ERR_INVALID_ARG, "expected %d parameters, got %d", (int)P.size(), n_params);
  for (int j = 0; j < n_params; ++j)
    if (!params[j]) return fail(VAEP_ERR_INVALID_ARG, "parameter %d (%s) is NULL", j, P[j].name.c_str());
  if ((rc = check_device())) return rc;
  hipStream_t st = (hipStream_t)stream;
  vaep_model* m = new (std::nothrow) vaep_model();
  if (!m) return fail(VAEP_ERR_INVALID_ARG, "out of host memory");
  m->cfg = *cfg;
  Builder sz{*cfg, params, {}, {}, st, true, cfg->dtype};
  for (size_t j = 0; j < P.size(); ++j) sz.index[P[j].name] = (int)j;
  sz.build(*m);
  m->mem_bytes = sz.carve.used;
  hipError_t e = hipMalloc(&m->mem, m->mem_bytes);
  if (e != hipSuccess) {
    delete m;
    return hip_fail(e, "hipMalloc(model)");
  }
  e = hipMemsetAsync(m->mem, 0, m->mem_bytes, st);
  Builder b{*cfg, params, sz.index, {}, st, false, cfg->dtype};
  b.carve.base = (char*)m->mem;
  b.build(*m);
  if (e == hipSuccess) e = b.err;
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    (void)hipFree(m->mem);
    delete m;
    return hip_fail(e, "model build");
  }
  *out = m;
  return VAEP_OK;
}

int vaep_model_destroy(vaep_model* model) {
  if (!model) return VAEP_OK;
  for (hipEvent_t ev : model->prof.ev) (void)hipEventDestroy(ev);
  hipError_t e = hipSuccess;
  if (model->mem) e = hipFree(model->mem);
  delete model;
  if (e != hipSuccess) return hip_fail(e, "hipFree(model)");
  return VAEP_OK;
}

int vaep_model_set_norm_fold(vaep_model* model, int on) {
  if (!model) return fail(VAEP_ERR_INVALID_ARG, "model is NULL");
  model->fold_norm = on ? 1 : 0;
  return VAEP_OK;
}

int vaep_model_set_halo_poison(vaep_model* model, int on) {
  if (!model) return fail(VAEP_ERR_INVALID_ARG, "model is NULL");
  model->poison_halos = on ? 1 : 0;
  return VAEP_OK;
}

int vaep_workspace_bytes(const vaep_model* model, int batch, int frames, int latent_h, int latent_w,
                         int n_bands, size_t* bytes_out) {
  int rc = check_latent_dims(model, batch, frames, latent_h, latent_w);
  if (rc) return rc;
  if (!bytes_out) return fail(VAEP_ERR_INVALID_ARG, "bytes_out is NULL");
  if (n_bands < 1) return fail(VAEP_ERR_INVALID_ARG, "n_bands must be >= 1");
  // row bands, and column bands of the same count (the larger of the two)
  size_t rows_b = 0, cols_b = 0;
  rc = plan_bytes(model, batch, frames, latent_h, latent_w, std::min(std::min(n_bands, kMaxBands), latent_h),
                  false, &rows_b);
  if (rc) return rc;
  rc = plan_bytes(model, batch, frames, latent_w, latent_h, std::min(std::min(n_bands, kMaxBands), latent_w),
                  true, &cols_b);
  if (rc) return rc;
  *bytes_out = std::max(rows_b, cols_b);
  return VAEP_OK;
}

int vaep_decode_bands(vaep_model* model, const void* latent, int batch, int frames, int latent_h,
                      int latent_w, const int32_t* row_starts, int n_bands, void* out, void* ws,
                      size_t ws_bytes, void* stream, vaep_decode_info* info) {
  int rc = check_latent_dims(model, batch, frames, latent_h, latent_w);
  if (rc) return rc;
  if (!latent || !out) return fail(VAEP_ERR_INVALID_ARG, "latent and out must be device pointers");
  if (!row_starts) return fail(VAEP_ERR_INVALID_ARG, "row_starts is NULL");
  if (n_bands < 1) return fail(VAEP_ERR_INVALID_ARG, "n_bands must be >= 1");
  std::vector<int> rows;
  if ((rc = table_rows(row_starts, n_bands, latent_h, "row", rows))) return rc;
  int status = VAEP_OK;
  if (n_bands > kMaxBands) {
    rows.assign(1, latent_h);      // dense fallback: one band
    status = VAEP_WARN_FELL_BACK;
  }
  rc = run_decode(model, latent, batch, frames, latent_w, false, rows,
                  status == VAEP_OK ? VAEP_AXIS_HEIGHT : VAEP_AXIS_DENSE, status, out, ws, ws_bytes, stream, info);
  if (rc) return rc;
  if (status == VAEP_WARN_FELL_BACK)
    fail(VAEP_WARN_FELL_BACK, "%d bands exceed the %d-band limit: decoded as one dense band", n_bands, kMaxBands);
  return status;
}

int vaep_tiled_workspace_bytes(const vaep_model* model, int batch, int frames, int latent_h, int latent_w,
                               int tile, int stride, size_t* bytes_out) {
  int rc = check_latent_dims(model, batch, frames, latent_h, latent_w);
  if (rc) return rc;
  if (!bytes_out) return fail(VAEP_ERR_INVALID_ARG, "bytes_out is NULL");
  TilePlan tp;
  if ((rc = tile_plan(model, batch, frames, latent_h, latent_w, tile, stride, &tp))) return rc;
  *bytes_out = tp.total;
  return VAEP_OK;
}

// The tile decode (split, decode every tile alone, blend, gather); arguments validated by
// the caller.  *launches receives the kernels enqueued, *tiles the tile count.
int tiled_decode(vaep_model* model, const void* latent, int batch, int frames, int latent_h, int latent_w,
                 int tile, int stride, void* out, void* ws, size_t ws_bytes, void* stream, int* launches,
                 int* tiles) {
  int rc;
  int n_launch = 0;
  vaep_decode_info sub{};
  TilePlan tp;
  if ((rc = tile_plan(model, batch, frames, latent_h, latent_w, tile, stride, &tp))) return rc;
  if (!ws || ws_bytes < tp.total)
    return fail(VAEP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", tp.total, ws ? ws_bytes : (size_t)0);
  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)ws;
  void* dec_ws = base;
  void* lat = base + tp.dec_bytes;
  float* stage = (float*)(base + tp.dec_bytes + tp.lat_bytes);
  float* slots = (float*)(base + tp.dec_bytes + tp.lat_bytes + tp.stage_bytes);
  const int cz = model->cfg.z_channels;
  const long long lat_planes = (long long)batch * cz * frames;
  // split / exec: every tile decoded on its own (its own statistics and attention), the
  // full-size ones together as a batch of images whose outputs land in consecutive slots
  // (the slots of full tiles are ordered first: slot k of the batch, then the edge tiles)
  std::vector<int> slot_of(tp.nr * tp.nc);
  for (int gi = 0; gi < tp.nr; ++gi)
    for (int gj = 0; gj < tp.nc; ++gj) slot_of[gi * tp.nc + gj] = tile_slot(gi, gj, tp.nc, tp.full_r, tp.full_c);
  const size_t lat_tile = (size_t)lat_planes * tile * tile * dtype_bytes(model->cfg.dtype);
  if (tp.nfull > 0) {
    for (int gi = 0; gi < tp.nr; ++gi)
      for (int gj = 0; gj < tp.nc; ++gj) {
        const int k = slot_of[gi * tp.nc + gj];
        if (k >= tp.nfull) continue;
        hipError_t e = launch_crop(latent, lat_planes, latent_h, latent_w, gi * stride, gj * stride, tile, tile,
                                   (char*)lat + k * lat_tile, model->cfg.dtype, st);
        if (e != hipSuccess) return hip_fail(e, "latent tile crop");
      }
    const std::vector<int> rows(1, tile);
    rc = run_decode(model, lat, batch * tp.nfull, frames, tile, false, rows, VAEP_AXIS_DENSE, VAEP_OK, slots, dec_ws,
                    tp.dec_bytes, stream, &sub);
    if (rc) return rc;
    n_launch += tp.nfull + sub.n_launches;
  }
  // the clipped edge tiles, one batch per size: decoded into the staging area, then each
  // tile's output copied to its slot
  for (const EdgeGroup& g : tp.edges) {
    const int n = (int)g.tiles.size();
    const size_t lat_g = (size_t)lat_planes * g.th * g.tw * dtype_bytes(model->cfg.dtype);
    for (int q = 0; q < n; ++q) {
      const int gi = g.tiles[q] / tp.nc, gj = g.tiles[q] % tp.nc;
      hipError_t e = launch_crop(latent, lat_planes, latent_h, latent_w, gi * stride, gj * stride, g.th, g.tw,
                                 (char*)lat + q * lat_g, model->cfg.dtype, st);
      if (e != hipSuccess) return hip_fail(e, "latent tile crop");
    }
    const std::vector<int> rows(1, g.th);
    rc = run_decode(model, lat, batch * n, frames, g.tw, false, rows, VAEP_AXIS_DENSE, VAEP_OK, stage, dec_ws,
                    tp.dec_bytes, stream, &sub);
    if (rc) return rc;
    n_launch += n + sub.n_launches;
    const size_t out_g = (size_t)tp.planes * g.th * tp.up * g.tw * tp.up;
    for (int q = 0; q < n; ++q) {
      hipError_t e = hipMemcpyAsync(slots + (long long)slot_of[g.tiles[q]] * tp.slot_elems, stage + q * out_g,
                                    out_g * sizeof(float), hipMemcpyDeviceToDevice, st);
      if (e != hipSuccess) return hip_fail(e, "tile output copy");
      ++n_launch;
    }
  }
  // merge: raster order, upper neighbour over the overlap rows, then left over the columns
  auto out_len = [&](int g, int len) { return std::min(tile, len - g * stride) * tp.up; };
  for (int gi = 0; gi < tp.nr; ++gi)
    for (int gj = 0; gj < tp.nc; ++gj) {
      float* t = slots + (long long)slot_of[gi * tp.nc + gj] * tp.slot_elems;
      const int th = out_len(gi, latent_h), tw = out_len(gj, latent_w);
      hipError_t e = hipSuccess;
      if (gi > 0) {
        const int uh = out_len(gi - 1, latent_h);
        e = launch_blend(slots + (long long)slot_of[(gi - 1) * tp.nc + gj] * tp.slot_elems, t, tp.planes, th, tw, uh,
                         std::min(std::min(uh, th), tp.blend), 0, st);
      }
      if (e == hipSuccess && gj > 0) {
        const int lw = out_len(gj - 1, latent_w);
        e = launch_blend(slots + (long long)slot_of[gi * tp.nc + gj - 1] * tp.slot_elems, t, tp.planes, th, tw, lw,
                         std::min(std::min(lw, tw), tp.blend), 1, st);
      }
      if (e != hipSuccess) return hip_fail(e, "tile blend");
      n_launch += (gi > 0) + (gj > 0);
    }
  hipError_t e = launch_tiles_gather(slots, tp.slot_elems, tp.planes, latent_h * tp.up, latent_w * tp.up,
                                     stride * tp.up, tile * tp.up, tp.nc, tp.full_r, tp.full_c, latent_h, latent_w,
                                     stride, tp.up, (float*)out, st);
  if (e != hipSuccess) return hip_fail(e, "tile gather");
  if (launches) *launches = n_launch + 1;
  if (tiles) *tiles = tp.nr * tp.nc;
  return VAEP_OK;
}

int vaep_decode_tiled(vaep_model* model, const void* latent, int batch, int frames, int latent_h, int latent_w,
                      int tile, int stride, void* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_latent_dims(model, batch, frames, latent_h, latent_w);
  if (rc) return rc;
  if (!latent || !out) return fail(VAEP_ERR_INVALID_ARG, "latent and out must be device pointers");
  return tiled_decode(model, latent, batch, frames, latent_h, latent_w, tile, stride, out, ws, ws_bytes, stream,
                      nullptr, nullptr);
}

int vaep_select_axis(int latent_h, int latent_w, int n_shards, int32_t* axis_out) {
  if (!axis_out) return fail(VAEP_ERR_INVALID_ARG, "axis_out is NULL");
  if (latent_h < 1 || latent_w < 1 || n_shards < 1)
    return fail(VAEP_ERR_INVALID_ARG, "latent %dx%d and n_shards %d must be >= 1", latent_h, latent_w, n_shards);
  *axis_out = select_axis(latent_h, latent_w, n_shards);
  return VAEP_OK;
}

int vaep_sharded_workspace_bytes(const vaep_model* model, int batch, int frames, int latent_h, int latent_w,
                                 int n_shards, size_t* bytes_out) {
  size_t bands = 0, tiles = 0;
  int rc = vaep_workspace_bytes(model, batch, frames, latent_h, latent_w, n_shards, &bands);
  if (rc) return rc;
  if ((rc = vaep_tiled_workspace_bytes(model, batch, frames, latent_h, latent_w, kShardTile, kShardTileStride, &tiles)))
    return rc;
  *bytes_out = std::max(bands, tiles);
  return VAEP_OK;
}

int vaep_decode_sharded(vaep_model* model, const void* latent, int batch, int frames, int latent_h,
                        int latent_w, int axis, const int32_t* starts, int n_shards, void* out, void* ws,
                        size_t ws_bytes, void* stream, vaep_decode_info* info) {
  int rc = check_latent_dims(model, batch, frames, latent_h, latent_w);
  if (rc) return rc;
  if (!latent || !out) return fail(VAEP_ERR_INVALID_ARG, "latent and out must be device pointers");
  if (n_shards < 1) return fail(VAEP_ERR_INVALID_ARG, "n_shards must be >= 1");
  if (axis != VAEP_AXIS_AUTO && axis != VAEP_AXIS_HEIGHT && axis != VAEP_AXIS_WIDTH && axis != VAEP_AXIS_TILE)
    return fail(VAEP_ERR_INVALID_ARG, "axis %d is not VAEP_AXIS_AUTO, _HEIGHT, _WIDTH or _TILE", axis);
  if ((axis == VAEP_AXIS_AUTO || axis == VAEP_AXIS_TILE) && starts)
    return fail(VAEP_ERR_INVALID_ARG, "VAEP_AXIS_AUTO and VAEP_AXIS_TILE take no shard table: starts must be NULL");
  int status = VAEP_OK;
  int chosen = axis;
  const char* why = nullptr;
  if (axis == VAEP_AXIS_AUTO) {
    chosen = select_axis(latent_h, latent_w, n_shards);
    if ((chosen == VAEP_AXIS_HEIGHT || chosen == VAEP_AXIS_WIDTH) && n_shards > kMaxBands) chosen = VAEP_AXIS_TILE;
  }
  std::vector<int> rows;
  if (chosen == VAEP_AXIS_HEIGHT || chosen == VAEP_AXIS_WIDTH) {
    const int len = chosen == VAEP_AXIS_WIDTH ? latent_w : latent_h;
    if (starts) {
      if ((rc = table_rows(starts, n_shards, len, chosen == VAEP_AXIS_WIDTH ? "column" : "row", rows))) return rc;
    } else if (len < n_shards) {
      why = "the axis is shorter than the shard count";
    } else {
      rows = even_rows(len, n_shards);
    }
    if (!why && n_shards > kMaxBands) why = "the shard count exceeds the band limit";
    if (why) {            // an explicit axis that cannot be honoured: warn and use the tile decode
      chosen = VAEP_AXIS_TILE;
      status = VAEP_WARN_FELL_BACK;
    }
  }
  if (chosen == VAEP_AXIS_TILE) {
    TilePlan tp;
    if ((rc = tile_plan(model, batch, frames, latent_h, latent_w, kShardTile, kShardTileStride, &tp))) return rc;
    if (!ws || ws_bytes < tp.total)
      return fail(VAEP_ERR_WORKSPACE, "the tile decode needs a workspace of %zu bytes (vaep_sharded_workspace_bytes), "
                                      "%zu given", tp.total, ws ? ws_bytes : (size_t)0);
    int launches = 0, tiles = 0;
    if ((rc = tiled_decode(model, latent, batch, frames, latent_h, latent_w, kShardTile, kShardTileStride, out, ws,
                           ws_bytes, stream, &launches, &tiles)))
      return rc;
    if (info) {
      info->bands_used = tiles;
      info->fell_back = axis != VAEP_AXIS_TILE;
      info->n_launches = launches;
      info->axis = VAEP_AXIS_TILE;
      info->workspace_bytes = tp.total;
    }
  } else {
    if (chosen == VAEP_AXIS_DENSE) rows.assign(1, latent_h);
    const bool tr = chosen == VAEP_AXIS_WIDTH;
    rc = run_decode(model, latent, batch, frames, tr ? latent_h : latent_w, tr, rows, chosen, status, out, ws,
                    ws_bytes, stream, info);
    if (rc) return rc;
    if (info) info->fell_back = 0;
  }
  if (status == VAEP_WARN_FELL_BACK)
    fail(VAEP_WARN_FELL_BACK, "%d shards along the %s: %s; decoded with the tile strategy", n_shards,
         axis == VAEP_AXIS_WIDTH ? "width" : "height", why);
  return status;
}

int vaep_decode_full(vaep_model* model, const void* latent, int batch, int frames, int latent_h,
                     int latent_w, void* out, void* ws, size_t ws_bytes, void* stream) {
  const int32_t starts[2] = {0, latent_h};
  return vaep_decode_bands(model, latent, batch, frames, latent_h, latent_w, starts, 1, out, ws,
                           ws_bytes, stream, nullptr);
}

int vaep_profile_begin(vaep_model* model, int max_launches) {
  if (!model) return fail(VAEP_ERR_INVALID_ARG, "model is NULL");
  if (max_launches < 1 || max_launches > (1 << 20)) return fail(VAEP_ERR_INVALID_ARG, "max_launches %d outside 1..2^20", max_launches);
  Profiler& p = model->prof;
  for (hipEvent_t e : p.ev) (void)hipEventDestroy(e);
  p.ev.clear();
  p.rec.clear();
  p.on = false;
  for (int i = 0; i < 2 * max_launches; ++i) {
    hipEvent_t e;
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      for (hipEvent_t x : p.ev) (void)hipEventDestroy(x);
      p.ev.clear();
      return hip_fail(r, "hipEventCreate");
    }
    p.ev.push_back(e);
  }
  p.cap = max_launches;
  p.on = true;
  return VAEP_OK;
}

int vaep_profile_end(vaep_model* model, vaep_profile_entry* out, int cap, int* n_out) {
  if (!model) return fail(VAEP_ERR_INVALID_ARG, "model is NULL");
  Profiler& p = model->prof;
  int rc = VAEP_OK;
  const int n = (int)p.rec.size();
  for (int i = 0; i < n; ++i) {
    float ms = 0.f;
    hipError_t r = hipEventSynchronize(p.ev[2 * i + 1]);
    if (r == hipSuccess) r = hipEventElapsedTime(&ms, p.ev[2 * i], p.ev[2 * i + 1]);
    if (r != hipSuccess && rc == VAEP_OK) rc = hip_fail(r, "profile events");
    p.rec[i].ms = ms;
    if (out && i < cap) out[i] = p.rec[i];
  }
  if (n_out) *n_out = n;
  for (hipEvent_t e : p.ev) (void)hipEventDestroy(e);
  p.ev.clear();
  p.rec.clear();
  p.on = false;
  p.cap = 0;
  return rc;
}

int vaep_groupnorm_merge(int n_shards, int n_stats, const float* local_mean, const float* local_var,
                         const int64_t* counts, float* mean_out, float* var_out, void* stream) {
  if (n_shards < 1 || n_shards > 4096) return fail(VAEP_ERR_INVALID_ARG, "n_shards %d outside 1..4096", n_shards);
  if (n_stats < 0) return fail(VAEP_ERR_INVALID_ARG, "n_stats must be >= 0");
  if (n_stats > 0 && (!local_mean || !local_var || !counts || !mean_out || !var_out))
    return fail(VAEP_ERR_INVALID_ARG, "NULL device pointer");
  hipError_t e = launch_moment_merge(n_shards, n_stats, local_mean, local_var, counts, mean_out, var_out,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "groupnorm merge launch");
  return VAEP_OK;
}

int vaep_step_conv(int dtype, int x_dtype, const void* x, int batch, int frames, int cin, int h,
                   int w, const void* weight, const void* bias, int cout, int kt, int kh, int kw,
                   int causal, int upsample, const void* residual, const int32_t* row_starts,
                   int n_bands, void* y, void* ws, size_t ws_bytes, size_t* bytes_out, void* stream) {
  int rc = step_dims(dtype, batch, frames, cin, h, w);
  if (rc) return rc;
  if (x_dtype != VAEP_DTYPE_F32 && x_dtype != dtype)
    return fail(VAEP_ERR_UNSUPPORTED, "x_dtype must be fp32 or the compute dtype");
  if (cout < 1) return fail(VAEP_ERR_INVALID_ARG, "cout must be >= 1");
  if (kh != kw || (kh != 1 && kh != 3)) return fail(VAEP_ERR_UNSUPPORTED, "spatial kernel %dx%d (1x1 or 3x3 only)", kh, kw);
  if (kt != 1 && kt != 3) return fail(VAEP_ERR_UNSUPPORTED, "temporal kernel %d (1 or 3 only)", kt);
  if (kt == 3 && !causal) return fail(VAEP_ERR_UNSUPPORTED, "a temporal kernel of 3 must be causal");
  if (kt == 3 && kh == 1) return fail(VAEP_ERR_UNSUPPORTED, "(3,1,1) convs run through vaep_step_temporal_upsample");
  if (upsample && (kt != 1 || kh != 3)) return fail(VAEP_ERR_UNSUPPORTED, "upsample fuses into 2-D 3x3 convs only");
  const bool bf = dtype == VAEP_DTYPE_BF16;
  if (bf && cout % 4 != 0) return fail(VAEP_ERR_UNSUPPORTED, "bf16 conv outputs need cout %% 4 == 0");
  std::vector<int> rows;
  if ((rc = step_bands(row_starts, n_bands, h, rows))) return rc;
  const int nb = (int)rows.size();
  const int cin_pad = bf ? round_up(cin, 32) : cin;
  const int co_pad = bf ? round_up(cout, kConvTileN) : cout;
  const int taps = kt * kh * kw;
  const BandLayout Lin = make_layout(nb, rows.data(), batch * frames, frames, w, cin_pad);
  const BandLayout Lout = upsample ? upsampled(Lin, cout) : reshaped(Lin, cout, Lin.n_img, frames);
  const size_t eb = dtype_bytes(dtype);
  const bool x_f32 = x_dtype == VAEP_DTYPE_F32;
  // bf16 upsample conv of an fp32 input: split the input into bf16 hi/lo parts and run the
  // sub-pixel form, as a decode does
  const bool sub = bf && upsample && x_f32 && cin % 64 == 0;
  const BandLayout Ls = reshaped(Lin, 2 * cin_pad, Lin.n_img, frames);
  Carver cv;
  cv.base = (char*)ws;
  void* xin = cv.take(layout_elems(Lin) * dtype_bytes(x_dtype));
  void* xs = sub ? cv.take(layout_elems(Ls) * 2) : nullptr;
  void* yo = cv.take(layout_elems(Lout) * 4);
  void* rb = residual ? cv.take(layout_elems(Lout) * 4) : nullptr;
  ConvW cw;
  cw.co = cout;
  cw.ci = cin;
  cw.co_pad = co_pad;
  cw.ci_pad = cin_pad;
  cw.kt = kt;
  cw.ks = kh;
  cw.w = cv.take((size_t)co_pad * taps * cin_pad * eb);
  cw.b = (float*)cv.take((size_t)co_pad * sizeof(float));
  if (sub) cw.wsub = cv.take((size_t)4 * co_pad * 4 * 2 * cin_pad * 2);
  if (sub) cw.sub_scale = (int*)cv.take(2 * sizeof(int));
  bool sized;
  if ((rc = step_finish_sizing(cv, ws, ws_bytes, bytes_out, &sized)) || sized) return rc;
  if (!x || !weight || !y) return fail(VAEP_ERR_INVALID_ARG, "x, weight and y must be device pointers");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_pack(x, cin, xin, Lin, x_dtype, st);
  if (e == hipSuccess && residual) e = launch_pack(residual, cout, rb, Lout, VAEP_DTYPE_F32, st);
  if (e == hipSuccess) e = launch_pack_weight(weight, cout, cin, taps, cw.w, co_pad, cin_pad, dtype, st);
  if (e == hipSuccess) e = launch_to_f32(bias, cout, cw.b, co_pad, dtype, st);
  if (e == hipSuccess && sub) e = launch_split((const float*)xin, Lin, xs, st);
  if (e == hipSuccess && sub) e = launch_fold_subpixel_weight(weight, cout, cin, cw.wsub, co_pad, cw.sub_scale, st);
  if (e != hipSuccess) return hip_fail(e, "step conv staging");
  Exec E;
  E.dtype = dtype;
  E.st = st;
  E.dry = false;
  if (sub) rc = E.conv(cw, xs, Ls, kXSplit, yo, Lout, kModeBand, rb, upsample);
  else rc = E.conv(cw, xin, Lin, x_f32 ? kXF32 : kXOp, yo, Lout, kModeBand, rb, upsample);
  if (rc) return rc;
  e = launch_unpack(yo, Lout, y, cout, VAEP_DTYPE_F32, st);
  if (e != hipSuccess) return hip_fail(e, "step conv gather");
  return VAEP_OK;
}

int vaep_step_groupnorm(int dtype, const void* x, int batch, int frames, int c, int h, int w, int groups,
                        float eps, const float* gamma, const float* beta, int act,
                        const int32_t* row_starts, int n_bands, void* y, float* band_moments,
                        float* merged, void* ws, size_t ws_bytes, size_t* bytes_out, void* stream) {
  int rc = step_dims(dtype, batch, frames, c, h, w);
  if (rc) return rc;
  if ((rc = norm_channels_ok(dtype, c))) return rc;
  if (groups < 1 || groups > 1024 || c % groups != 0) return fail(VAEP_ERR_INVALID_ARG, "groups %d must divide %d (<= 1024)", groups, c);
  if (!(eps > 0.f)) return fail(VAEP_ERR_INVALID_ARG, "eps must be > 0");
  std::vector<int> rows;
  if ((rc = step_bands(row_starts, n_bands, h, rows))) return rc;
  const int nb = (int)rows.size();
  const BandLayout L = make_layout(nb, rows.data(), batch * frames, frames, w, c);
  const size_t eb = dtype_bytes(dtype);
  Carver cv;
  cv.base = (char*)ws;
  void* xin = cv.take(layout_elems(L) * 4);
  void* yo = cv.take(layout_elems(L) * eb);
  float* scratch = (float*)cv.take(gn_partials_floats(L, groups, 1) * sizeof(float));
  bool sized;
  if ((rc = step_finish_sizing(cv, ws, ws_bytes, bytes_out, &sized)) || sized) return rc;
  if (!x || !y || !gamma || !beta) return fail(VAEP_ERR_INVALID_ARG, "x, y, gamma and beta must be device pointers");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_pack(x, c, xin, L, VAEP_DTYPE_F32, st);
  if (e != hipSuccess) return hip_fail(e, "step groupnorm staging");
  NormArgs a;
  std::memset(&a, 0, sizeof(a));
  a.x = xin;
  a.y = yo;
  a.L = L;
  a.groups = groups;
  a.eps = eps;
  a.gamma = gamma;
  a.beta = beta;
  a.act = act;
  a.partials = reinterpret_cast<double*>(scratch);
  a.merged_out = merged;
  a.slab_rows = 1;
  a.want_band_moments = band_moments ? 1 : 0;
  e = launch_groupnorm(a, dtype, st);
  if (e == hipSuccess && band_moments)
    e = hipMemcpyAsync(band_moments, a.band_moments, sizeof(float) * 3 * nb * L.n_img * groups,
                       hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess) e = launch_unpack(yo, L, y, c, dtype, st);
  if (e != hipSuccess) return hip_fail(e, "step groupnorm");
  return VAEP_OK;
}

int vaep_step_rmsnorm(int dtype, const void* x, int batch, int frames, int c, int h, int w, float eps,
                      const float* gamma, int act, const int32_t* row_starts, int n_bands, void* y,
                      void* ws, size_t ws_bytes, size_t* bytes_out, void* stream) {
  int rc = step_dims(dtype, batch, frames, c, h, w);
  if (rc) return rc;
  if ((rc = norm_channels_ok(dtype, c))) return rc;
  if (!(eps > 0.f)) return fail(VAEP_ERR_INVALID_ARG, "eps must be > 0");
  std::vector<int> rows;
  if ((rc = step_bands(row_starts, n_bands, h, rows))) return rc;
  const int nb = (int)rows.size();
  const BandLayout L = make_layout(nb, rows.data(), batch * frames, frames, w, c);
  const size_t eb = dtype_bytes(dtype);
  Carver cv;
  cv.base = (char*)ws;
  void* xin = cv.take(layout_elems(L) * 4);
  void* yo = cv.take(layout_elems(L) * eb);
  bool sized;
  if ((rc = step_finish_sizing(cv, ws, ws_bytes, bytes_out, &sized)) || sized) return rc;
  if (!x || !y || !gamma) return fail(VAEP_ERR_INVALID_ARG, "x, y and gamma must be device pointers");
  hipStream_t st = (hipStream_t)stream;
  NormArgs a;
  std::memset(&a, 0, sizeof(a));
  a.x = xin;
  a.y = yo;
  a.L = L;
  a.eps = eps;
  a.gamma = gamma;
  a.act = act;
  hipError_t e = launch_pack(x, c, xin, L, VAEP_DTYPE_F32, st);
  if (e == hipSuccess) e = launch_rmsnorm(a, dtype, st);
  if (e == hipSuccess) e = launch_unpack(yo, L, y, c, dtype, st);
  if (e != hipSuccess) return hip_fail(e, "step rmsnorm");
  return VAEP_OK;
}

int vaep_step_attention(int dtype, const void* x, int batch, int frames, int c, int h, int w, int groups,
                        float eps, const float* norm_gamma, const float* norm_beta, const void* wq,
                        const void* bq, const void* wk, const void* bk, const void* wv, const void* bv,
                        const void* wo, const void* bo, const int32_t* row_starts, int n_bands, void* y,
                        void* ws, size_t ws_bytes, size_t* bytes_out, void* stream) {
  int rc = step_dims(dtype, batch, frames, c, h, w);
  if (rc) return rc;
  if ((rc = norm_channels_ok(dtype, c))) return rc;
  const bool bf = dtype == VAEP_DTYPE_BF16;
  if (bf && c != 128 && c != 256 && c != 384 && c != 512)
    return fail(VAEP_ERR_UNSUPPORTED, "bf16 attention supports 128/256/384/512 channels, got %d", c);
  if (groups < 0 || (groups > 0 && (groups > 1024 || c % groups != 0)))
    return fail(VAEP_ERR_INVALID_ARG, "groups %d must divide %d", groups, c);
  if (!(eps > 0.f)) return fail(VAEP_ERR_INVALID_ARG, "eps must be > 0");
  std::vector<int> rows;
  if ((rc = step_bands(row_starts, n_bands, h, rows))) return rc;
  const int nb = (int)rows.size();
  const BandLayout L = make_layout(nb, rows.data(), batch * frames, frames, w, c);
  const size_t eb = dtype_bytes(dtype);
  Carver cv;
  cv.base = (char*)ws;
  void* bufs[4];  // x (fp32), normalised x, attention output (operand dtype), y (fp32)
  for (int i = 0; i < 4; ++i) bufs[i] = cv.take(layout_elems(L) * ((i == 0 || i == 3) ? 4 : eb));
  const size_t qkv = (size_t)L.n_img * h * w * c * eb;
  void* qb = cv.take(qkv);
  void* kb = cv.take(qkv);
  void* vb = cv.take(qkv);
  // statistics records, and the key-split attention's halves (bf16)
  const long long sc_floats = std::max<long long>(groups > 0 ? (long long)gn_partials_floats(L, groups, 1) : 0,
                                                  bf ? attn_part_floats(L.n_img, h * w, c) : 0);
  float* scratch = sc_floats > 0 ? (float*)cv.take((size_t)sc_floats * sizeof(float)) : nullptr;
  AttnW aw;
  aw.norm.g = const_cast<float*>(norm_gamma);
  aw.norm.b = const_cast<float*>(norm_beta);
  aw.norm.c = c;
  aw.qkv.co = 3 * c;
  aw.qkv.ci = c;
  aw.qkv.co_pad = bf ? round_up(3 * c, kConvTileN) : 3 * c;
  aw.qkv.ci_pad = c;
  aw.qkv.kt = 1;
  aw.qkv.ks = 1;
  aw.qkv.w = cv.take((size_t)aw.qkv.co_pad * c * eb);
  aw.qkv.b = (float*)cv.take((size_t)aw.qkv.co_pad * sizeof(float));
  aw.out = aw.qkv;
  aw.out.co = c;
  aw.out.co_pad = bf ? round_up(c, kConvTileN) : c;
  aw.out.w = cv.take((size_t)aw.out.co_pad * c * eb);
  aw.out.b = (float*)cv.take((size_t)aw.out.co_pad * sizeof(float));
  bool sized;
  if ((rc = step_finish_sizing(cv, ws, ws_bytes, bytes_out, &sized)) || sized) return rc;
  if (!x || !y || !norm_gamma || (groups > 0 && !norm_beta) || !wq || !wk || !wv || !wo)
    return fail(VAEP_ERR_INVALID_ARG, "NULL device pointer");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipMemsetAsync(aw.qkv.w, 0, (size_t)aw.qkv.co_pad * c * eb, st);
  const void* ws_[3] = {wq, wk, wv};
  const void* bs_[3] = {bq, bk, bv};
  for (int i = 0; i < 3 && e == hipSuccess; ++i) {
    e = launch_pack_weight(ws_[i], c, c, 1, (char*)aw.qkv.w + (size_t)i * c * c * eb, c, c, dtype, st);
    if (e == hipSuccess) e = launch_to_f32(bs_[i], c, aw.qkv.b + (size_t)i * c, c, dtype, st);
  }
  if (e == hipSuccess) e = launch_to_f32(nullptr, 0, aw.qkv.b + 3 * c, aw.qkv.co_pad - 3 * c, dtype, st);
  if (e == hipSuccess) e = launch_pack_weight(wo, c, c, 1, aw.out.w, aw.out.co_pad, c, dtype, st);
  if (e == hipSuccess) e = launch_to_f32(bo, c, aw.out.b, aw.out.co_pad, dtype, st);
  if (e == hipSuccess) e = launch_pack(x, c, bufs[0], L, VAEP_DTYPE_F32, st);
  if (e != hipSuccess) return hip_fail(e, "step attention staging");
  Exec E;
  E.dtype = dtype;
  E.st = st;
  E.dry = false;
  E.groups = groups;
  E.eps = eps;
  E.qb = qb;
  E.kb = kb;
  E.vb = vb;
  E.scratch = scratch;
  if ((rc = E.attention(aw, bufs[0], L, bufs[1], bufs[2], bufs[3]))) return rc;
  e = launch_unpack(bufs[3], L, y, c, VAEP_DTYPE_F32, st);
  if (e != hipSuccess) return hip_fail(e, "step attention gather");
  return VAEP_OK;
}

int vaep_step_temporal_upsample(int dtype, const void* x, int batch, int frames, int c, int h, int w,
                                const void* weight, const void* bias, const int32_t* row_starts,
                                int n_bands, void* y, void* ws, size_t ws_bytes, size_t* bytes_out,
                                void* stream) {
  int rc = step_dims(dtype, batch, frames, c, h, w);
  if (rc) return rc;
  const bool bf = dtype == VAEP_DTYPE_BF16;
  if (bf && c % 32 != 0) return fail(VAEP_ERR_UNSUPPORTED, "bf16 temporal upsample needs c %% 32 == 0");
  std::vector<int> rows;
  if ((rc = step_bands(row_starts, n_bands, h, rows))) return rc;
  const int nb = (int)rows.size();
  const int T2 = 2 * frames - 1;
  const BandLayout Lx = make_layout(nb, rows.data(), batch * frames, frames, w, c);
  const BandLayout Lt = reshaped(Lx, c, batch * T2, T2);
  const size_t eb = dtype_bytes(dtype);
  Carver cv;
  cv.base = (char*)ws;
  void* xin = cv.take(layout_elems(Lx) * 4);
  void* yo = cv.take(layout_elems(Lt) * 4);
  ConvW cw;
  cw.co = 2 * c;
  cw.ci = c;
  cw.co_pad = bf ? round_up(2 * c, kConvTileN) : 2 * c;
  cw.ci_pad = c;
  cw.kt = 3;
  cw.ks = 1;
  cw.w = cv.take((size_t)cw.co_pad * 3 * c * eb);
  cw.b = (float*)cv.take((size_t)cw.co_pad * sizeof(float));
  bool sized;
  if ((rc = step_finish_sizing(cv, ws, ws_bytes, bytes_out, &sized)) || sized) return rc;
  if (!x || !y || !weight) return fail(VAEP_ERR_INVALID_ARG, "x, weight and y must be device pointers");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_pack(x, c, xin, Lx, VAEP_DTYPE_F32, st);
  if (e == hipSuccess) e = launch_pack_weight(weight, 2 * c, c, 3, cw.w, cw.co_pad, c, dtype, st);
  if (e == hipSuccess) e = launch_to_f32(bias, 2 * c, cw.b, cw.co_pad, dtype, st);
  if (e != hipSuccess) return hip_fail(e, "step temporal upsample staging");
  Exec E;
  E.dtype = dtype;
  E.st = st;
  E.dry = false;
  if ((rc = E.conv(cw, xin, Lx, kXF32, yo, Lt, kModeTimeInterleave, nullptr, 0))) return rc;
  e = launch_copy_frame0(xin, Lx, yo, Lt, VAEP_DTYPE_F32, st);
  if (e == hipSuccess) e = launch_unpack(yo, Lt, y, c, VAEP_DTYPE_F32, st);
  if (e != hipSuccess) return hip_fail(e, "step temporal upsample");
  return VAEP_OK;
}

// ------------------------------------------------------------------ tiled encode

int vaep_encoder_param_count(const vaep_config* cfg) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (is_video(*cfg)) return fail(VAEP_ERR_UNSUPPORTED, "the encoder is built for the 2-D family only");
  return (int)encoder_param_list(*cfg).size();
}

int vaep_encoder_param_info(const vaep_config* cfg, int j, char* name, int name_cap, int64_t shape[5], int* ndim) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (is_video(*cfg)) return fail(VAEP_ERR_UNSUPPORTED, "the encoder is built for the 2-D family only");
  const auto P = encoder_param_list(*cfg);
  if (j < 0 || j >= (int)P.size()) return fail(VAEP_ERR_INVALID_ARG, "parameter index %d outside 0..%d", j, (int)P.size() - 1);
  if (name && name_cap > 0) {
    std::strncpy(name, P[j].name.c_str(), name_cap - 1);
    name[name_cap - 1] = 0;
  }
  if (shape)
    for (size_t i = 0; i < P[j].shape.size() && i < 5; ++i) shape[i] = P[j].shape[i];
  if (ndim) *ndim = (int)P[j].shape.size();
  return VAEP_OK;
}

int vaep_encoder_create(const vaep_config* cfg, const void* const* params, int n_params, void* stream,
                        vaep_encoder** out) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (is_video(*cfg)) return fail(VAEP_ERR_UNSUPPORTED, "the encoder is built for the 2-D family only");
  if (!out) return fail(VAEP_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  const auto P = encoder_param_list(*cfg);
  if (!params) return fail(VAEP_ERR_INVALID_ARG, "params is NULL");
  if (n_params != (int)P.size()) return fail(VAEP_ERR_INVALID_ARG, "expected %d parameters, got %d", (int)P.size(), n_params);
  for (int j = 0; j < n_params; ++j)
    if (!params[j]) return fail(VAEP_ERR_INVALID_ARG, "parameter %d (%s) is NULL", j, P[j].name.c_str());
  if ((rc = check_device())) return rc;
  hipStream_t st = (hipStream_t)stream;
  vaep_encoder* e = new (std::nothrow) vaep_encoder();
  if (!e) return fail(VAEP_ERR_INVALID_ARG, "out of host memory");
  e->cfg = *cfg;
  Builder sz{*cfg, params, {}, {}, st, true, cfg->dtype};
  for (size_t j = 0; j < P.size(); ++j) sz.index[P[j].name] = (int)j;
  sz.build_encoder(*e);
  e->mem_bytes = sz.carve.used;
  hipError_t err = hipMalloc(&e->mem, e->mem_bytes);
  if (err != hipSuccess) {
    delete e;
    return hip_fail(err, "hipMalloc(encoder)");
  }
  err = hipMemsetAsync(e->mem, 0, e->mem_bytes, st);
  Builder b{*cfg, params, sz.index, {}, st, false, cfg->dtype};
  b.carve.base = (char*)e->mem;
  b.build_encoder(*e);
  if (err == hipSuccess) err = b.err;
  if (err == hipSuccess) err = hipStreamSynchronize(st);
  if (err != hipSuccess) {
    (void)hipFree(e->mem);
    delete e;
    return hip_fail(err, "encoder build");
  }
  *out = e;
  return VAEP_OK;
}

int vaep_encoder_destroy(vaep_encoder* enc) {
  if (!enc) return VAEP_OK;
  hipError_t e = enc->mem ? hipFree(enc->mem) : hipSuccess;
  delete enc;
  return e == hipSuccess ? VAEP_OK : hip_fail(e, "hipFree(encoder)");
}

int vaep_encode_tiled_workspace_bytes(const vaep_encoder* enc, int batch, int height, int width, int tile,
                                      int stride, size_t* bytes_out) {
  int rc = check_image_dims(enc, batch, height, width);
  if (rc) return rc;
  if (!bytes_out) return fail(VAEP_ERR_INVALID_ARG, "bytes_out is NULL");
  EncTilePlan tp;
  if ((rc = enc_tile_plan(enc, batch, height, width, tile, stride, &tp))) return rc;
  *bytes_out = tp.total;
  return VAEP_OK;
}

int vaep_encode_tiled(vaep_encoder* enc, const void* image, int batch, int height, int width, int tile, int stride,
                      void* out, void* ws, size_t ws_bytes, void* stream, vaep_decode_info* info) {
  int rc = check_image_dims(enc, batch, height, width);
  if (rc) return rc;
  if (!image || !out) return fail(VAEP_ERR_INVALID_ARG, "image and out must be device pointers");
  EncTilePlan tp;
  if ((rc = enc_tile_plan(enc, batch, height, width, tile, stride, &tp))) return rc;
  if (!ws || ws_bytes < tp.total)
    return fail(VAEP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", tp.total, ws ? ws_bytes : (size_t)0);
  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)ws;
  void* enc_ws = base;
  void* img = base + tp.enc_bytes;
  float* stage = (float*)(base + tp.enc_bytes + tp.img_bytes);
  float* slots = (float*)(base + tp.enc_bytes + tp.img_bytes + tp.stage_bytes);
  const int up = tp.up, dt = enc->cfg.dtype;
  const long long img_planes = (long long)batch * 3;
  int n_launch = 0;
  std::vector<int> slot_of(tp.nr * tp.nc);
  for (int gi = 0; gi < tp.nr; ++gi)
    for (int gj = 0; gj < tp.nc; ++gj) slot_of[gi * tp.nc + gj] = tile_slot(gi, gj, tp.nc, tp.full_r, tp.full_c);
  // split / exec: every tile encoded on its own; the full-size tiles together as one batch
  // of images whose moments land in consecutive slots, the clipped edge tiles one batch per size
  const int ts = tile * up;
  const size_t img_tile = (size_t)img_planes * ts * ts * dtype_bytes(dt);
  if (tp.nfull > 0) {
    for (int gi = 0; gi < tp.nr; ++gi)
      for (int gj = 0; gj < tp.nc; ++gj) {
        const int k = slot_of[gi * tp.nc + gj];
        if (k >= tp.nfull) continue;
        hipError_t e = launch_crop(image, img_planes, height, width, gi * stride * up, gj * stride * up, ts, ts,
                                   (char*)img + k * img_tile, dt, st);
        if (e != hipSuccess) return hip_fail(e, "image tile crop");
        ++n_launch;
      }
    if ((rc = run_encode(enc, img, batch * tp.nfull, ts, ts, slots, enc_ws, tp.enc_bytes, stream, &n_launch)))
      return rc;
  }
  for (const EdgeGroup& g : tp.edges) {
    const int n = (int)g.tiles.size();
    const int th = g.th * up, tw = g.tw * up;
    const size_t img_g = (size_t)img_planes * th * tw * dtype_bytes(dt);
    for (int q = 0; q < n; ++q) {
      const int gi = g.tiles[q] / tp.nc, gj = g.tiles[q] % tp.nc;
      hipError_t e = launch_crop(image, img_planes, height, width, gi * stride * up, gj * stride * up, th, tw,
                                 (char*)img + q * img_g, dt, st);
      if (e != hipSuccess) return hip_fail(e, "image tile crop");
      ++n_launch;
    }
    if ((rc = run_encode(enc, img, batch * n, th, tw, stage, enc_ws, tp.enc_bytes, stream, &n_launch))) return rc;
    const size_t out_g = (size_t)tp.planes * g.th * g.tw;
    for (int q = 0; q < n; ++q) {
      hipError_t e = hipMemcpyAsync(slots + (long long)slot_of[g.tiles[q]] * tp.slot_elems, stage + q * out_g,
                                    out_g * sizeof(float), hipMemcpyDeviceToDevice, st);
      if (e != hipSuccess) return hip_fail(e, "tile moments copy");
      ++n_launch;
    }
  }
  // merge in latent space: raster order, upper neighbour over the overlap rows, then left
  auto len = [&](int g, int n) { return std::min(tile, n - g * stride); };
  const int blend = tile - stride;
  for (int gi = 0; gi < tp.nr; ++gi)
    for (int gj = 0; gj < tp.nc; ++gj) {
      float* t = slots + (long long)slot_of[gi * tp.nc + gj] * tp.slot_elems;
      const int th = len(gi, tp.lh), tw = len(gj, tp.lw);
      hipError_t e = hipSuccess;
      if (gi > 0) {
        const int uh = len(gi - 1, tp.lh);
        e = launch_blend(slots + (long long)slot_of[(gi - 1) * tp.nc + gj] * tp.slot_elems, t, tp.planes, th, tw, uh,
                         std::min(std::min(uh, th), blend), 0, st);
      }
      if (e == hipSuccess && gj > 0) {
        const int lw = len(gj - 1, tp.lw);
        e = launch_blend(slots + (long long)slot_of[gi * tp.nc + gj - 1] * tp.slot_elems, t, tp.planes, th, tw, lw,
                         std::min(std::min(lw, tw), blend), 1, st);
      }
      if (e != hipSuccess) return hip_fail(e, "tile blend");
      n_launch += (gi > 0) + (gj > 0);
    }
  hipError_t e = launch_tiles_gather(slots, tp.slot_elems, tp.planes, tp.lh, tp.lw, stride, tile, tp.nc, tp.full_r,
                                     tp.full_c, tp.lh, tp.lw, stride, 1, (float*)out, st);
  if (e != hipSuccess) return hip_fail(e, "tile gather");
  if (info) {
    info->bands_used = tp.nr * tp.nc;
    info->fell_back = 0;
    info->n_launches = n_launch + 1;
    info->axis = VAEP_AXIS_TILE;
    info->workspace_bytes = tp.total;
  }
  return VAEP_OK;
}

}  // extern "C"
