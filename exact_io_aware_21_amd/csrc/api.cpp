// C-ABI layer of libattn.so: argument validation, device check, workspace layout and dispatch.
// Declarations and the contract of each entry point are in include/attn.h.
#include "attn.h"

#include <hip/hip_runtime.h>
#include <hip/hiprtc.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "launch.h"

namespace {

thread_local char g_err[256] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

constexpr uint32_t kKnownBits = 0xFu | ATTN_MOD_ALIBI | ATTN_MOD_SOFTCAP | ATTN_PREC_FP8;
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other
char g_arch_name[kMaxDevices][64];         // written before g_arch_ok is set to -1

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Shape {
  int B, H, N, d, n_qt, n_kt, Npad, Bm;
  uint32_t kind;
  bool fp8;
};

// Validates the shape and variant bits; fills s.  No HIP call.
int check_shape(int B, int H, int N, int d, uint32_t variant, Shape &s) {
  if (B < 1 || H < 1 || N < 1) return fail(ATTN_ERR_INVALID_ARG, "B, H and N must be >= 1");
  if (N > (1 << 24)) return fail(ATTN_ERR_INVALID_ARG, "N must be <= 2^24");
  if (d != 64 && d != 128 && d != 256) return fail(ATTN_ERR_INVALID_ARG, "d must be 64, 128 or 256");
  // The kernels address a V^T tile with 32-bit per-lane offsets of up to (columns of O - 1) *
  // Npad * 2 bytes: below 2^31 for 64 columns up to N = 2^24, for 128 up to N = 2^23.
  if (d >= 128 && N > (1 << 23))
    return fail(ATTN_ERR_INVALID_ARG, "N must be <= 2^23 for d 128 and 256");
  if (variant & ~kKnownBits) return fail(ATTN_ERR_INVALID_ARG, "unknown variant bits");
  s.kind = variant & 0xFu;
  if (s.kind > ATTN_MASK_DOCUMENT) return fail(ATTN_ERR_INVALID_ARG, "unknown mask kind");
  s.fp8 = (variant & ATTN_PREC_FP8) != 0;
  if (s.fp8 && d == 256) return fail(ATTN_ERR_INVALID_ARG, "ATTN_PREC_FP8 takes d 64 or 128");
  if (s.fp8 && (variant & (ATTN_MOD_ALIBI | ATTN_MOD_SOFTCAP)))
    return fail(ATTN_ERR_INVALID_ARG, "ATTN_PREC_FP8 takes no score modification");
  if (s.fp8 && (long long)B * H > 65535)
    return fail(ATTN_ERR_INVALID_ARG, "B*H must be <= 65535 with ATTN_PREC_FP8");
  s.B = B;
  s.H = H;
  s.N = N;
  s.d = d;
  s.n_qt = (N + attn::kBr - 1) / attn::kBr;
  s.n_kt = (N + attn::kBc - 1) / attn::kBc;
  s.Npad = s.n_kt * attn::kBc;
  s.Bm = s.kind == ATTN_MASK_DOCUMENT ? B : 1;
  if ((long long)B * H * s.n_qt >= (1ll << 31))
    return fail(ATTN_ERR_INVALID_ARG, "B*H*ceil(N/Br) must be < 2^31");
  return ATTN_OK;
}

// Validates the params fields the variant uses.  No HIP call.
int check_params(const Shape &s, uint32_t variant, const attn_params *p, bool need_ws) {
  if (!p) {
    if (need_ws || s.kind == ATTN_MASK_SLIDING_WINDOW || s.kind == ATTN_MASK_DOCUMENT ||
        (variant & (ATTN_MOD_ALIBI | ATTN_MOD_SOFTCAP)))
      return fail(ATTN_ERR_INVALID_ARG, "params is NULL");
    return ATTN_OK;
  }
  if (s.kind == ATTN_MASK_SLIDING_WINDOW && p->window < 1)
    return fail(ATTN_ERR_INVALID_ARG, "window must be >= 1");
  if (s.kind == ATTN_MASK_DOCUMENT) {
    if (!p->doc_offsets) return fail(ATTN_ERR_INVALID_ARG, "doc_offsets is NULL");
    if (p->max_docs < 1) return fail(ATTN_ERR_INVALID_ARG, "max_docs must be >= 1");
    if ((uintptr_t)p->doc_offsets % 4) return fail(ATTN_ERR_INVALID_ARG, "doc_offsets misaligned");
  }
  if (variant & ATTN_MOD_SOFTCAP) {
    if (!(p->softcap > 0.f) || !std::isfinite(p->softcap))
      return fail(ATTN_ERR_INVALID_ARG, "softcap must be finite and > 0");
  }
  if (variant & ATTN_MOD_ALIBI) {
    if (!p->alibi_slopes) return fail(ATTN_ERR_INVALID_ARG, "alibi_slopes is NULL");
    if ((uintptr_t)p->alibi_slopes % 4) return fail(ATTN_ERR_INVALID_ARG, "alibi_slopes misaligned");
  }
  if (p->o_dtype != ATTN_O_BF16 && p->o_dtype != ATTN_O_F32)
    return fail(ATTN_ERR_INVALID_ARG, "o_dtype must be ATTN_O_BF16 or ATTN_O_F32");
  return ATTN_OK;
}

struct WsLayout {
  size_t vt, cls, cnt, list, k8, sk, total;
};

WsLayout ws_layout(const Shape &s) {
  WsLayout w{};
  size_t off = 0;
  w.vt = off;
  off = align256(off + (size_t)s.B * s.H * s.d * s.Npad * 2);
  if (s.kind != ATTN_MASK_NONE) {
    const size_t rows = (size_t)s.Bm * s.n_qt;
    w.cls = off;
    off = align256(off + rows * s.n_kt);
    w.cnt = off;
    off = align256(off + rows * 4);
    w.list = off;
    off = align256(off + rows * s.n_kt * 4);
  }
  if (s.fp8) {
    w.k8 = off;
    off = align256(off + (size_t)s.B * s.H * s.N * s.d);
    w.sk = off;
    off = align256(off + (size_t)s.B * s.H * s.n_kt * 4);
  }
  w.total = off;
  return w;
}

// Backward workspace: D (fp32 [BH][N]) and, for masked kinds, the forward block table.
struct BwdLayout {
  size_t dvec, cls, cnt, list, total;
};

BwdLayout bwd_layout(const Shape &s) {
  BwdLayout w{};
  size_t off = 0;
  w.dvec = off;
  off = align256(off + (size_t)s.B * s.H * s.N * 4);
  if (s.kind != ATTN_MASK_NONE) {
    const size_t rows = (size_t)s.Bm * s.n_qt;
    w.cls = off;
    off = align256(off + rows * s.n_kt);
    w.cnt = off;
    off = align256(off + rows * 4);
    w.list = off;
    off = align256(off + rows * s.n_kt * 4);
  }
  w.total = off;
  return w;
}

// Paged decoding: shape check and the split plan.  A split covers keys_per_split consecutive
// positions (a multiple of the G = 256 / (d / 8) rows of a chunk).  The lengths live on the
// device, so the plan is made for the longest possible sequence: about 8192 workgroups over all
// (sequence, head) pairs when every sequence has that length (shorter ones leave their trailing
// splits empty; those exit at once), and no split shorter than 256 positions.
struct DecodePlan {
  int lq_pad, rows, keys_per_split, nsplit;
  size_t part_o, part_m, part_l, total;  // workspace offsets and size
};

int decode_plan(int B, int H, int Lq, int d, int page, int max_pages, DecodePlan &p) {
  if (B < 1 || H < 1) return fail(ATTN_ERR_INVALID_ARG, "B and H must be >= 1");
  if ((long long)B * H > 65535) return fail(ATTN_ERR_INVALID_ARG, "B*H must be <= 65535");
  if (Lq < 1 || Lq > 8) return fail(ATTN_ERR_INVALID_ARG, "Lq must be in [1, 8]");
  if (d != 64 && d != 128) return fail(ATTN_ERR_INVALID_ARG, "d must be 64 or 128");
  p.rows = 256 / (d / 8);
  if (page < p.rows || page > 4096 || (page & (page - 1)))
    return fail(ATTN_ERR_INVALID_ARG, "page_size must be a power of two in [%d, 4096]", p.rows);
  if (max_pages < 1 || (long long)max_pages * page > (1 << 24))
    return fail(ATTN_ERR_INVALID_ARG, "max_pages must be >= 1 with max_pages*page_size <= 2^24");
  p.lq_pad = Lq <= 1 ? 1 : Lq <= 2 ? 2 : Lq <= 4 ? 4 : 8;
  const long long max_len = (long long)max_pages * page;
  const long long bh = (long long)B * H;
  long long ns = (8192 + bh - 1) / bh;
  const long long ns_max = (max_len + 255) / 256;
  if (ns > ns_max) ns = ns_max;
  if (ns > 65535) ns = 65535;  // grid dimension
  if (ns < 1) ns = 1;
  long long kps = (max_len + ns - 1) / ns;
  kps = (kps + p.rows - 1) / p.rows * p.rows;
  p.keys_per_split = (int)kps;
  p.nsplit = (int)((max_len + kps - 1) / kps);
  const size_t nparts = (size_t)bh * p.nsplit * p.lq_pad;
  size_t off = 0;
  p.part_o = off;
  off = align256(off + nparts * d * 4);
  p.part_m = off;
  off = align256(off + nparts * 4);
  p.part_l = off;
  off = align256(off + nparts * 4);
  p.total = off;
  return ATTN_OK;
}

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(ATTN_ERR_UNSUPPORTED_DEVICE, "no HIP device available");
  }
  if (dev < kMaxDevices) {
    const int c = g_arch_ok[dev].load(std::memory_order_acquire);
    if (c == 1) return ATTN_OK;
    if (c == -1)
      return fail(ATTN_ERR_UNSUPPORTED_DEVICE, "device %d is %s, not gfx950", dev,
                  g_arch_name[dev]);
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(ATTN_ERR_UNSUPPORTED_DEVICE, "cannot query device %d", dev);
  }
  // Test hook: ATTN_TEST_ARCH_OVERRIDE, if set when a device is first checked, stands in for the
  // architecture name the device reports, so that the unsupported-device path can be exercised
  // on a gfx950 (nothing is launched on that path).
  const char *ov = std::getenv("ATTN_TEST_ARCH_OVERRIDE");
  const char *arch = (ov && *ov) ? ov : prop.gcnArchName;
  const bool ok = std::strncmp(arch, "gfx950", 6) == 0;
  if (dev < kMaxDevices) {
    if (!ok) std::snprintf(g_arch_name[dev], sizeof g_arch_name[dev], "%s", arch);
    g_arch_ok[dev].store(ok ? 1 : -1, std::memory_order_release);
  }
  if (!ok) return fail(ATTN_ERR_UNSUPPORTED_DEVICE, "device %d is %s, not gfx950", dev, arch);
  return ATTN_OK;
}

attn::MaskDesc mask_desc(const Shape &s, const attn_params *p) {
  attn::MaskDesc m{};
  m.kind = (int)s.kind;
  m.N = s.N;
  m.window = (p && s.kind == ATTN_MASK_SLIDING_WINDOW) ? p->window : 0;
  m.offs = nullptr;
  m.max_docs = (p && s.kind == ATTN_MASK_DOCUMENT) ? p->max_docs : 0;
  return m;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// ---------------------------------------------------------------------------------------------
// Runtime-compiled score / mask modifications (attn_mod_*).  The kernel headers are embedded in
// the library (rtc_sources.s); hipRTC compiles them with the user's source into a gfx950 code
// object, which each device loads on first use.
extern "C" const char attn_rtc_hipdefs_h[], attn_rtc_kcommon_h[], attn_rtc_tiles_h[],
    attn_rtc_launch_h[], attn_rtc_fwd_kernel_h[];

struct ModLayout {
  size_t vt, cls, cnt, list, wfull, total;
};

ModLayout mod_layout(const Shape &s, bool mask) {
  ModLayout w{};
  size_t off = 0;
  w.vt = off;
  off = align256(off + (size_t)s.B * s.H * s.d * s.Npad * 2);
  if (mask) {
    const size_t rows = (size_t)s.B * s.n_qt;
    w.cls = off;
    off = align256(off + rows * s.n_kt);
    w.cnt = off;
    off = align256(off + rows * 4);
    w.list = off;
    off = align256(off + rows * s.n_kt * 4);
    w.wfull = off;
    off = align256(off + rows * s.n_kt);
  }
  w.total = off;
  return w;
}

}  // namespace

struct attn_mod_s {
  std::string code;  // gfx950 code object
  uint32_t flags = 0;
  int d = 0;
  std::mutex mu;
  hipModule_t module[kMaxDevices] = {};
  hipFunction_t fwd[kMaxDevices][2] = {};  // bf16 O, fp32 O
  hipFunction_t cls[kMaxDevices] = {}, list[kMaxDevices] = {};
};

namespace {

// The code object of m loaded on device dev (once), its kernels in m's per-device tables.
int mod_load(attn_mod *m, int dev) {
  std::lock_guard<std::mutex> g(m->mu);
  if (m->module[dev]) return ATTN_OK;
  hipModule_t mod = nullptr;
  if (hipModuleLoadData(&mod, m->code.data()) != hipSuccess) {
    (void)hipGetLastError();
    return fail(ATTN_ERR_LAUNCH, "loading the compiled modification on device %d failed", dev);
  }
  hipFunction_t f16 = nullptr, f32 = nullptr, fc = nullptr, fl = nullptr;
  bool ok = hipModuleGetFunction(&f16, mod, "attn_mod_fwd_bf16") == hipSuccess &&
            hipModuleGetFunction(&f32, mod, "attn_mod_fwd_f32") == hipSuccess;
  if (ok && (m->flags & ATTN_MODF_MASK))
    ok = hipModuleGetFunction(&fc, mod, "attn_mod_class") == hipSuccess &&
         hipModuleGetFunction(&fl, mod, "attn_mod_list") == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    (void)hipModuleUnload(mod);
    return fail(ATTN_ERR_LAUNCH, "compiled modification lacks its kernels");
  }
  m->fwd[dev][0] = f16;
  m->fwd[dev][1] = f32;
  m->cls[dev] = fc;
  m->list[dev] = fl;
  m->module[dev] = mod;
  return ATTN_OK;
}

void copy_log(const char *text, char *log, size_t log_size) {
  if (!log || log_size == 0) return;
  std::snprintf(log, log_size, "%s", text ? text : "");
}

}  // namespace

extern "C" {

const char *attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case ATTN_ERR_COMPILE: return "runtime compilation of the modification failed";
    default: return "unknown error code";
  }
}

const char *attn_last_error(void) { return g_err; }

int attn_tile_shape(int d, uint32_t variant, int *Br, int *Bc) {
  if (d != 64 && d != 128 && d != 256)
    return fail(ATTN_ERR_INVALID_ARG, "d must be 64, 128 or 256");
  if ((variant & ATTN_PREC_FP8) && d == 256)
    return fail(ATTN_ERR_INVALID_ARG, "ATTN_PREC_FP8 takes d 64 or 128");
  if (variant & ~kKnownBits || (variant & 0xFu) > ATTN_MASK_DOCUMENT)
    return fail(ATTN_ERR_INVALID_ARG, "unknown variant bits");
  if (!Br || !Bc) return fail(ATTN_ERR_INVALID_ARG, "Br/Bc output pointer is NULL");
  *Br = attn::kBr;
  *Bc = attn::kBc;
  return ATTN_OK;
}

size_t attn_workspace_size(int B, int H, int N, int d, uint32_t variant) {
  Shape s;
  if (check_shape(B, H, N, d, variant, s) != ATTN_OK) return 0;
  return ws_layout(s).total;
}

int attn_block_table_host(int B, int H, int N, int d, uint32_t variant, const attn_params *params,
                          int8_t *cls, int32_t *kv_cnt, int32_t *kv_list) {
  Shape s;
  int rc = check_shape(B, H, N, d, variant, s);
  if (rc) return rc;
  // the table depends only on the mask kind: score modifications are not validated here
  if ((rc = check_params(s, variant & 0xFu, params, false))) return rc;
  if (!cls || !kv_cnt || !kv_list) return fail(ATTN_ERR_INVALID_ARG, "output pointer is NULL");
  attn::MaskDesc m = mask_desc(s, params);
  for (int bm = 0; bm < s.Bm; ++bm) {
    if (s.kind == ATTN_MASK_DOCUMENT) m.offs = params->doc_offsets + (size_t)bm * (m.max_docs + 1);
    for (int qt = 0; qt < s.n_qt; ++qt) {
      const size_t row = (size_t)bm * s.n_qt + qt;
      kv_cnt[row] = attn::tile_row(m, qt, s.n_kt, attn::kBr, attn::kBc, cls + row * s.n_kt,
                                   kv_list + row * s.n_kt);
    }
  }
  return ATTN_OK;
}

int attn_block_table(int B, int H, int N, int d, uint32_t variant, const attn_params *params,
                     int8_t *cls, int32_t *kv_cnt, int32_t *kv_list, void *stream) {
  Shape s;
  int rc = check_shape(B, H, N, d, variant, s);
  if (rc) return rc;
  // the table depends only on the mask kind: score modifications are not validated here
  if ((rc = check_params(s, variant & 0xFu, params, false))) return rc;
  if (!cls || !kv_cnt || !kv_list) return fail(ATTN_ERR_INVALID_ARG, "output pointer is NULL");
  if (((uintptr_t)kv_cnt | (uintptr_t)kv_list) & 3u)
    return fail(ATTN_ERR_INVALID_ARG, "kv_cnt/kv_list misaligned");
  if ((rc = check_device())) return rc;
  const attn::MaskDesc m = mask_desc(s, params);
  const int32_t *offs = s.kind == ATTN_MASK_DOCUMENT ? params->doc_offsets : nullptr;
  if (attn::launch_block_table(m, offs, s.Bm, s.n_qt, s.n_kt, cls, kv_cnt, kv_list,
                               (hipStream_t)stream) != hipSuccess)
    return fail(ATTN_ERR_LAUNCH, "block table kernel launch failed");
  return ATTN_OK;
}

}  // extern "C"

namespace {

// Validation of attn_fwd's arguments other than the workspace (no HIP call); fills s.
int fwd_check(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
              int N, int d, float scale, uint32_t variant, const attn_params *params, Shape &s) {
  int rc = check_shape(B, H, N, d, variant, s);
  if (rc) return rc;
  if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (lse && ((uintptr_t)lse & 3u)) return fail(ATTN_ERR_INVALID_ARG, "lse misaligned");
  if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
  return check_params(s, variant, params, false);
}

// Which kernel takes a forward pass: the tiled kernel (V^T pack and block table, then key tiles
// walked per 256-row query tile), or for short sequences the single-launch kernel, which holds
// all N <= 256 keys of a head in LDS (K and V^T: up to 137 KB per workgroup at N = 256,
// d = 128) and re-reads them per 64 query rows.  Measured against the tiled kernel on one
// MI355X (device time per call from graph replays), the short kernel is as fast or faster for
// d = 64 and for N <= 128 at every grid measured (B H up to 2048), and for d = 128 with
// 128 < N <= 256 while the grid has at most 256 workgroups (its 137 KB of LDS allow one
// workgroup per CU); beyond that the tiled kernel's throughput wins.  ATTN_FWD_PATH=tiled|short overrides the choice (for tests and
// measurements); "short" on a shape the short kernel does not take is an error.
int fwd_short_path(const Shape &s, bool &use_short) {
  const bool fits = !s.fp8 && s.d <= 128 && s.N <= attn::kShortMaxN;
  const char *env = std::getenv("ATTN_FWD_PATH");
  if (env && *env) {
    if (!std::strcmp(env, "tiled")) {
      use_short = false;
      return ATTN_OK;
    }
    if (!std::strcmp(env, "short")) {
      if (!fits)
        return fail(ATTN_ERR_INVALID_ARG,
                    "ATTN_FWD_PATH=short takes N <= %d, d 64 or 128 and bf16 operands",
                    attn::kShortMaxN);
      use_short = true;
      return ATTN_OK;
    }
    return fail(ATTN_ERR_INVALID_ARG, "ATTN_FWD_PATH must be 'tiled' or 'short', not '%s'", env);
  }
  const long long wgs = (long long)s.B * s.H * ((s.N + 63) / 64);
  use_short = fits && (s.d == 64 || s.N <= 128 || wgs <= 256);
  return ATTN_OK;
}

// The launches of one forward pass on validated arguments, with the workspace at ws (at least
// ws_layout(s).total bytes).  Launches only: allocates nothing.
int fwd_launch(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
               int N, int d, float scale, uint32_t variant, const attn_params *params,
               const Shape &s, char *ws, hipStream_t st) {
  bool use_short = false;
  int rc = fwd_short_path(s, use_short);
  if (rc) return rc;
  const WsLayout wl = ws_layout(s);
  uint16_t *vt = (uint16_t *)(ws + wl.vt);
  attn::FwdArgs a{};
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.v = (const uint16_t *)v;
  a.vt = vt;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.N = N;
  a.Npad = s.Npad;
  a.n_qt = s.n_qt;
  a.n_kt = s.n_kt;
  const float log2e = 1.4426950408889634f;
  a.c = scale * log2e;
  if (variant & ATTN_MOD_SOFTCAP) {
    a.cap_c1 = 2.f * scale * log2e / params->softcap;
    a.capL = params->softcap * log2e;
  }
  a.slopes = (variant & ATTN_MOD_ALIBI) ? params->alibi_slopes : nullptr;
  a.kind = (int)s.kind;
  a.window = s.kind == ATTN_MASK_SLIDING_WINDOW ? params->window : 0;
  a.max_docs = s.kind == ATTN_MASK_DOCUMENT ? params->max_docs : 0;
  a.offs = s.kind == ATTN_MASK_DOCUMENT ? params->doc_offsets : nullptr;
  attn::FwdInstance in{};
  in.d = d;
  in.alibi = (variant & ATTN_MOD_ALIBI) != 0;
  in.softcap = (variant & ATTN_MOD_SOFTCAP) != 0;
  in.pos_scale = !in.alibi && !in.softcap && scale > 0.f;
  in.out_f32 = params->o_dtype == ATTN_O_F32;
  in.fp8 = s.fp8;
  void *const *ev = params->timing_events;
  if (use_short) {
    if (ev && hipEventRecord((hipEvent_t)ev[0], st) != hipSuccess)
      return fail(ATTN_ERR_LAUNCH, "timing event record failed");
    if (attn::launch_fwd_short(in, a, st) != hipSuccess)
      return fail(ATTN_ERR_LAUNCH, "short-sequence forward kernel launch failed");
    if (ev && hipEventRecord((hipEvent_t)ev[1], st) != hipSuccess)
      return fail(ATTN_ERR_LAUNCH, "timing event record failed");
    return ATTN_OK;
  }
  if (s.fp8) {
    // K to E4M3 codes with one scale per 64-key tile; Q is quantized inside the forward kernel.
    uint8_t *k8 = (uint8_t *)(ws + wl.k8);
    float *sk = (float *)(ws + wl.sk);
    if (attn::launch_quant_fp8((const uint16_t *)k, k8, sk, B * H, N, d, attn::kBc, st) !=
        hipSuccess)
      return fail(ATTN_ERR_LAUNCH, "FP8 quantization kernel launch failed");
    a.k8 = k8;
    a.sk = sk;
  }
  if (s.kind != ATTN_MASK_NONE) {
    a.cls = (const int8_t *)(ws + wl.cls);
    a.cnt = (const int32_t *)(ws + wl.cnt);
    a.list = (const int32_t *)(ws + wl.list);
  }
  // V^T pack and block table: one launch
  if (attn::launch_prep((const uint16_t *)v, vt, B * H, N, s.Npad, d, mask_desc(s, params), a.offs,
                        s.Bm, s.n_qt, s.n_kt, (int8_t *)a.cls, (int32_t *)a.cnt,
                        (int32_t *)a.list, st) != hipSuccess)
    return fail(ATTN_ERR_LAUNCH, "V transpose / block table kernel launch failed");
  if (ev && hipEventRecord((hipEvent_t)ev[0], st) != hipSuccess)
    return fail(ATTN_ERR_LAUNCH, "timing event record failed");
  if (attn::launch_fwd(in, a, st) != hipSuccess)
    return fail(ATTN_ERR_LAUNCH, "forward kernel launch failed");
  if (ev && hipEventRecord((hipEvent_t)ev[1], st) != hipSuccess)
    return fail(ATTN_ERR_LAUNCH, "timing event record failed");
  return ATTN_OK;
}

// ---------------------------------------------------------------------------------------------
// The workspace of attn_fwd_noalloc: a file-scope device array (each device holds its own copy
// from the library's load on it until the process ends).  In host code `scratch` only names the
// symbol; its device address is resolved once per device with hipGetSymbolAddress, with that
// device current, and only that address is ever handed to a kernel.
constexpr size_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
char *g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (resolved on the device's first call).
int scratch_on_current_device(char **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return fail(ATTN_ERR_UNSUPPORTED_DEVICE, "no usable current device");
  }
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(ATTN_ERR_LAUNCH, "resolving the static scratch array on device %d failed", dev);
    }
    if ((uintptr_t)p & 255u)
      return fail(ATTN_ERR_LAUNCH, "the static scratch array is not 256-byte aligned");
    g_scratch_ptr[dev] = (char *)p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int N,
             int d, float scale, uint32_t variant, const attn_params *params, void *stream) {
  Shape s;
  int rc = fwd_check(q, k, v, o, lse, B, H, N, d, scale, variant, params, s);
  if (rc) return rc;
  if (!params) return fail(ATTN_ERR_INVALID_ARG, "params is NULL");
  const WsLayout wl = ws_layout(s);
  if (!params->workspace || ((uintptr_t)params->workspace & 255u))
    return fail(ATTN_ERR_WORKSPACE, "workspace is NULL or not 256-byte aligned");
  if (params->workspace_bytes < wl.total)
    return fail(ATTN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", params->workspace_bytes,
                wl.total);
  if ((rc = check_device())) return rc;
  return fwd_launch(q, k, v, o, lse, B, H, N, d, scale, variant, params, s,
                    (char *)params->workspace, (hipStream_t)stream);
}

int attn_fwd_noalloc(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                     int H, int N, int d, float scale, uint32_t variant,
                     const attn_params *params, void *stream) {
  Shape s;
  int rc = fwd_check(q, k, v, o, lse, B, H, N, d, scale, variant, params, s);
  if (rc) return rc;
  if (!params) return fail(ATTN_ERR_INVALID_ARG, "params is NULL");
  const size_t need = ws_layout(s).total;
  if (need > kScratchBytes)
    return fail(ATTN_ERR_WORKSPACE,
                "this shape needs %zu bytes of workspace; the static scratch holds %zu "
                "(use attn_fwd with a caller workspace)", need, kScratchBytes);
  if ((rc = check_device())) return rc;
  char *ws = nullptr;
  if ((rc = scratch_on_current_device(&ws))) return rc;
  return fwd_launch(q, k, v, o, lse, B, H, N, d, scale, variant, params, s, ws,
                    (hipStream_t)stream);
}

size_t attn_bwd_workspace_size(int B, int H, int N, int d, uint32_t variant) {
  Shape s;
  if (check_shape(B, H, N, d, variant, s) != ATTN_OK || s.fp8 || d == 256) return 0;
  return bwd_layout(s).total;
}

int attn_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
             const void *dout, void *dq, void *dk, void *dv, int B, int H, int N, int d,
             float scale, uint32_t variant, const attn_params *params, void *stream) {
  Shape s;
  int rc = check_shape(B, H, N, d, variant, s);
  if (rc) return rc;
  if (s.fp8) return fail(ATTN_ERR_INVALID_ARG, "ATTN_PREC_FP8 is a forward-only variant");
  if (d == 256) return fail(ATTN_ERR_INVALID_ARG, "the backward pass takes d 64 or 128");
  if ((long long)B * H > 65535) return fail(ATTN_ERR_INVALID_ARG, "B*H must be <= 65535");
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
    return fail(ATTN_ERR_INVALID_ARG, "q, k, v, o, lse, dout, dq, dk and dv must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(ATTN_ERR_INVALID_ARG, "tensor arguments must be 16-byte aligned");
  if ((uintptr_t)lse & 3u) return fail(ATTN_ERR_INVALID_ARG, "lse misaligned");
  if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
  if ((rc = check_params(s, variant, params, true))) return rc;
  const BwdLayout wl = bwd_layout(s);
  if (!params->workspace || ((uintptr_t)params->workspace & 255u))
    return fail(ATTN_ERR_WORKSPACE, "workspace is NULL or not 256-byte aligned");
  if (params->workspace_bytes < wl.total)
    return fail(ATTN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", params->workspace_bytes,
                wl.total);
  if ((rc = check_device())) return rc;

  const hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)params->workspace;
  attn::BwdArgs a{};
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.v = (const uint16_t *)v;
  a.dout = (const uint16_t *)dout;
  a.o = o;
  a.lse = lse;
  a.dvec = (float *)(ws + wl.dvec);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.H = H;
  a.N = N;
  a.Npad = s.Npad;
  a.n_qt = s.n_qt;
  a.n_kt = s.n_kt;
  const float log2e = 1.4426950408889634f;
  a.scale = scale;
  a.c = scale * log2e;
  if (variant & ATTN_MOD_SOFTCAP) {
    a.cap_c1 = 2.f * scale * log2e / params->softcap;
    a.capL = params->softcap * log2e;
  }
  a.slopes = (variant & ATTN_MOD_ALIBI) ? params->alibi_slopes : nullptr;
  a.kind = (int)s.kind;
  a.window = s.kind == ATTN_MASK_SLIDING_WINDOW ? params->window : 0;
  a.max_docs = s.kind == ATTN_MASK_DOCUMENT ? params->max_docs : 0;
  a.offs = s.kind == ATTN_MASK_DOCUMENT ? params->doc_offsets : nullptr;
  a.o_f32 = a.out_f32 = params->o_dtype == ATTN_O_F32;

  if (attn::launch_bwd_dot(a, d, st) != hipSuccess)
    return fail(ATTN_ERR_LAUNCH, "row-dot kernel launch failed");
  if (s.kind != ATTN_MASK_NONE) {
    a.cnt = (const int32_t *)(ws + wl.cnt);
    a.list = (const int32_t *)(ws + wl.list);
    if (attn::launch_block_table(mask_desc(s, params), a.offs, s.Bm, s.n_qt, s.n_kt,
                                 (int8_t *)(ws + wl.cls), (int32_t *)(ws + wl.cnt),
                                 (int32_t *)(ws + wl.list), st) != hipSuccess)
      return fail(ATTN_ERR_LAUNCH, "block table kernel launch failed");
  }
  void *const *ev = params->timing_events;
  if (ev && hipEventRecord((hipEvent_t)ev[0], st) != hipSuccess)
    return fail(ATTN_ERR_LAUNCH, "timing event record failed");
  if (attn::launch_bwd(a, d, (variant & ATTN_MOD_ALIBI) != 0, (variant & ATTN_MOD_SOFTCAP) != 0,
                       st) != hipSuccess)
    return fail(ATTN_ERR_LAUNCH, "backward kernel launch failed");
  if (ev && hipEventRecord((hipEvent_t)ev[1], st) != hipSuccess)
    return fail(ATTN_ERR_LAUNCH, "timing event record failed");
  return ATTN_OK;
}

int attn_quantize_fp8(const void *x, uint8_t *codes, float *scales, int B, int H, int N, int d,
                      int rows, void *stream) {
  if (B < 1 || H < 1 || N < 1) return fail(ATTN_ERR_INVALID_ARG, "B, H and N must be >= 1");
  if ((long long)B * H > 65535) return fail(ATTN_ERR_INVALID_ARG, "B*H must be <= 65535");
  if (N > (1 << 24)) return fail(ATTN_ERR_INVALID_ARG, "N must be <= 2^24");
  if (d != 64 && d != 128) return fail(ATTN_ERR_INVALID_ARG, "d must be 64 or 128");
  if (rows < 1 || rows > 4096) return fail(ATTN_ERR_INVALID_ARG, "rows must be in [1, 4096]");
  if (!x || !codes || !scales)
    return fail(ATTN_ERR_INVALID_ARG, "x, codes and scales must be non-NULL");
  if (!aligned16(x) || !aligned16(codes))
    return fail(ATTN_ERR_INVALID_ARG, "x and codes must be 16-byte aligned");
  if ((uintptr_t)scales & 3u) return fail(ATTN_ERR_INVALID_ARG, "scales misaligned");
  int rc = check_device();
  if (rc) return rc;
  if (attn::launch_quant_fp8((const uint16_t *)x, codes, scales, B * H, N, d, rows,
                             (hipStream_t)stream) != hipSuccess)
    return fail(ATTN_ERR_LAUNCH, "quantization kernel launch failed");
  return ATTN_OK;
}

size_t attn_decode_workspace_size(int B, int H, int Lq, int d, int page_size, int max_pages) {
  DecodePlan p;
  if (decode_plan(B, H, Lq, d, page_size, max_pages, p) != ATTN_OK) return 0;
  return p.total;
}

int attn_decode(const void *q, const void *k_cache, const void *v_cache,
                const int32_t *page_table, const int32_t *seq_lens, void *o, float *lse, int B,
                int H, int Lq, int d, int page_size, int max_pages, int n_pages, float scale,
                uint32_t variant, const attn_params *params, void *stream) {
  DecodePlan p;
  int rc = decode_plan(B, H, Lq, d, page_size, max_pages, p);
  if (rc) return rc;
  if (n_pages < 1) return fail(ATTN_ERR_INVALID_ARG, "n_pages must be >= 1");
  if (variant != ATTN_MASK_NONE && variant != ATTN_MASK_CAUSAL)
    return fail(ATTN_ERR_INVALID_ARG, "decode supports ATTN_MASK_NONE and ATTN_MASK_CAUSAL only");
  if (!q || !k_cache || !v_cache || !page_table || !seq_lens || !o)
    return fail(ATTN_ERR_INVALID_ARG, "q, k_cache, v_cache, page_table, seq_lens and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(ATTN_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be 16-byte aligned");
  if (((uintptr_t)page_table | (uintptr_t)seq_lens | (uintptr_t)lse) & 3u)
    return fail(ATTN_ERR_INVALID_ARG, "page_table, seq_lens or lse misaligned");
  if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
  if (!params) return fail(ATTN_ERR_INVALID_ARG, "params is NULL");
  if (params->o_dtype != ATTN_O_BF16 && params->o_dtype != ATTN_O_F32)
    return fail(ATTN_ERR_INVALID_ARG, "unknown o_dtype");
  if (!params->workspace || ((uintptr_t)params->workspace & 255u))
    return fail(ATTN_ERR_WORKSPACE, "workspace is NULL or not 256-byte aligned");
  if (params->workspace_bytes < p.total)
    return fail(ATTN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", params->workspace_bytes,
                p.total);
  if ((rc = check_device())) return rc;

  const hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)params->workspace;
  attn::DecodeArgs a{};
  a.q = (const uint16_t *)q;
  a.k_cache = (const uint16_t *)k_cache;
  a.v_cache = (const uint16_t *)v_cache;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.o = o;
  a.lse = lse;
  a.part_o = (float *)(ws + p.part_o);
  a.part_m = (float *)(ws + p.part_m);
  a.part_l = (float *)(ws + p.part_l);
  a.B = B;
  a.H = H;
  a.Lq = Lq;
  a.lq_pad = p.lq_pad;
  a.page = page_size;
  a.max_pages = max_pages;
  a.n_pages = n_pages;
  a.keys_per_split = p.keys_per_split;
  a.nsplit = p.nsplit;
  a.causal = variant == ATTN_MASK_CAUSAL;
  a.c = scale * 1.4426950408889634f;
  void *const *ev = params->timing_events;
  if (ev && hipEventRecord((hipEvent_t)ev[0], st) != hipSuccess)
    return fail(ATTN_ERR_LAUNCH, "timing event record failed");
  if (attn::launch_decode(a, d, params->o_dtype == ATTN_O_F32, st) != hipSuccess)
    return fail(ATTN_ERR_LAUNCH, "decode kernel launch failed");
  if (ev && hipEventRecord((hipEvent_t)ev[1], st) != hipSuccess)
    return fail(ATTN_ERR_LAUNCH, "timing event record failed");
  return ATTN_OK;
}

}  // extern "C"

namespace {

int mod_create(const char *source, uint32_t flags, int d, attn_mod **out, char *log,
               size_t log_size) {
  copy_log("", log, log_size);
  if (!out) return fail(ATTN_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!source) return fail(ATTN_ERR_INVALID_ARG, "source is NULL");
  if (!(flags & (ATTN_MODF_SCORE | ATTN_MODF_MASK)) ||
      (flags & ~(uint32_t)(ATTN_MODF_SCORE | ATTN_MODF_MASK | ATTN_MODF_MAX_FIRST)))
    return fail(ATTN_ERR_INVALID_ARG,
                "flags must hold ATTN_MODF_SCORE and/or ATTN_MODF_MASK (optionally with "
                "ATTN_MODF_MAX_FIRST) and nothing else");
  if (d != 64 && d != 128 && d != 256)
    return fail(ATTN_ERR_INVALID_ARG, "d must be 64, 128 or 256");
  std::string prog = "#include \"fwd_kernel.h\"\n#line 1 \"attn_mod_source\"\n";
  prog += source;
  char tail[1024];
  std::snprintf(tail, sizeof tail,
                "\n#line 1 \"attn_mod_kernels\"\n"
                "extern \"C\" __global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))"
                " void attn_mod_fwd_bf16(attn::FwdArgs a) {"
                " attn::fwd_body<%d, false, false, true, false, false, %u>(a); }\n"
                "extern \"C\" __global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))"
                " void attn_mod_fwd_f32(attn::FwdArgs a) {"
                " attn::fwd_body<%d, false, false, true, true, false, %u>(a); }\n",
                d, flags, d, flags);
  prog += tail;
  if (flags & ATTN_MODF_MASK)
    prog +=
        "extern \"C\" __global__ __launch_bounds__(256) void attn_mod_class(attn::ModTableArgs t) {"
        " attn::mod_class_body(t); }\n"
        "extern \"C\" __global__ __launch_bounds__(256) void attn_mod_list(attn::ModTableArgs t) {"
        " attn::mod_list_body(t); }\n";
  const char *hdrs[] = {attn_rtc_hipdefs_h, attn_rtc_kcommon_h, attn_rtc_tiles_h, attn_rtc_launch_h,
                        attn_rtc_fwd_kernel_h};
  const char *names[] = {"hipdefs.h", "kcommon.h", "tiles.h", "launch.h", "fwd_kernel.h"};
  hiprtcProgram p;
  if (hiprtcCreateProgram(&p, prog.c_str(), "attn_mod.hip", 5, hdrs, names) != HIPRTC_SUCCESS)
    return fail(ATTN_ERR_COMPILE, "hiprtcCreateProgram failed");
  // Packed fp32 VALU instructions are disabled, as for the library's own kernels.
  const char *opts[] = {"--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops"};
  const hiprtcResult rc = hiprtcCompileProgram(p, 7, opts);
  size_t n = 0;
  std::vector<char> text(1, 0);
  if (hiprtcGetProgramLogSize(p, &n) == HIPRTC_SUCCESS && n > 0) {
    text.assign(n + 1, 0);
    (void)hiprtcGetProgramLog(p, text.data());
  }
  copy_log(text.data(), log, log_size);
  if (rc != HIPRTC_SUCCESS) {
    (void)hiprtcDestroyProgram(&p);
    return fail(ATTN_ERR_COMPILE, "compilation failed: %.200s", text.data());
  }
  size_t cs = 0;
  std::string code;
  if (hiprtcGetCodeSize(p, &cs) == HIPRTC_SUCCESS && cs > 0) {
    code.resize(cs);
    if (hiprtcGetCode(p, &code[0]) != HIPRTC_SUCCESS) code.clear();
  }
  (void)hiprtcDestroyProgram(&p);
  if (code.empty()) return fail(ATTN_ERR_COMPILE, "no code object produced");
  attn_mod *m = new attn_mod;
  m->code = std::move(code);
  m->flags = flags;
  m->d = d;
  *out = m;
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_mod_create(const char *source, uint32_t flags, int d, attn_mod **out, char *log,
                    size_t log_size) {
  try {  // the C ABI does not throw: host allocation failures become an error code
    return mod_create(source, flags, d, out, log, log_size);
  } catch (...) {
    if (out) *out = nullptr;
    return fail(ATTN_ERR_COMPILE, "host memory exhausted while compiling the modification");
  }
}

void attn_mod_destroy(attn_mod *m) {
  if (!m) return;
  int cur = -1;
  const bool have = hipGetDevice(&cur) == hipSuccess;
  for (int dev = 0; dev < kMaxDevices; ++dev) {
    if (!m->module[dev]) continue;
    if (hipSetDevice(dev) == hipSuccess) (void)hipModuleUnload(m->module[dev]);
  }
  if (have) (void)hipSetDevice(cur);
  (void)hipGetLastError();
  delete m;
}

size_t attn_mod_workspace_size(const attn_mod *m, int B, int H, int N) {
  if (!m) return 0;
  Shape s;
  if (check_shape(B, H, N, m->d, ATTN_MASK_NONE, s) != ATTN_OK) return 0;
  if ((long long)B * s.n_qt > 65535 && (m->flags & ATTN_MODF_MASK)) return 0;
  return mod_layout(s, (m->flags & ATTN_MODF_MASK) != 0).total;
}

}  // extern "C"

namespace {

int fwd_mod(const attn_mod *mc, const void *q, const void *k, const void *v, void *o, float *lse,
            int B, int H, int N, float scale, const float *mod_params,
            const attn_params *params, void *stream, bool build_table) {
  attn_mod *m = const_cast<attn_mod *>(mc);
  if (!m) return fail(ATTN_ERR_INVALID_ARG, "mod is NULL");
  const int d = m->d;
  Shape s;
  int rc = check_shape(B, H, N, d, ATTN_MASK_NONE, s);
  if (rc) return rc;
  const bool mask = (m->flags & ATTN_MODF_MASK) != 0;
  if (mask && (long long)B * s.n_qt > 65535)
    return fail(ATTN_ERR_INVALID_ARG, "B*ceil(N/Br) must be <= 65535 with a mask modification");
  if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (lse && ((uintptr_t)lse & 3u)) return fail(ATTN_ERR_INVALID_ARG, "lse misaligned");
  if ((uintptr_t)mod_params & 3u) return fail(ATTN_ERR_INVALID_ARG, "mod_params misaligned");
  if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
  if (!params) return fail(ATTN_ERR_INVALID_ARG, "params is NULL");
  if (params->o_dtype != ATTN_O_BF16 && params->o_dtype != ATTN_O_F32)
    return fail(ATTN_ERR_INVALID_ARG, "o_dtype must be ATTN_O_BF16 or ATTN_O_F32");
  const ModLayout wl = mod_layout(s, mask);
  if (!params->workspace || ((uintptr_t)params->workspace & 255u))
    return fail(ATTN_ERR_WORKSPACE, "workspace is NULL or not 256-byte aligned");
  if (params->workspace_bytes < wl.total)
    return fail(ATTN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", params->workspace_bytes,
                wl.total);
  if ((rc = check_device())) return rc;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(ATTN_ERR_UNSUPPORTED_DEVICE, "device index out of range");
  if ((rc = mod_load(m, dev))) return rc;

  const hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)params->workspace;
  uint16_t *vt = (uint16_t *)(ws + wl.vt);
  if (attn::launch_vt_pack((const uint16_t *)v, vt, B * H, N, s.Npad, d, st) != hipSuccess)
    return fail(ATTN_ERR_LAUNCH, "V transpose kernel launch failed");
  attn::FwdArgs a{};
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.vt = vt;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.N = N;
  a.Npad = s.Npad;
  a.n_qt = s.n_qt;
  a.n_kt = s.n_kt;
  a.c = 1.4426950408889634f;  // scores reach the softmax in natural units (see fwd_kernel.h)
  a.scale = scale;
  a.mod_params = mod_params;
  a.kind = ATTN_MASK_NONE;
  if (mask) {  // the block table: built here, or left by an earlier call (build_table false)
    attn::ModTableArgs t{};
    t.N = N;
    t.n_qt = s.n_qt;
    t.n_kt = s.n_kt;
    t.params = mod_params;
    t.cls = (int8_t *)(ws + wl.cls);
    t.cnt = (int32_t *)(ws + wl.cnt);
    t.list = (int32_t *)(ws + wl.list);
    t.wfull = (uint8_t *)(ws + wl.wfull);
    void *targs[] = {&t};
    if (build_table &&
        (hipModuleLaunchKernel(m->cls[dev], (unsigned)s.n_kt, (unsigned)(B * s.n_qt), 1, 256, 1,
                               1, 0, st, targs, nullptr) != hipSuccess ||
         hipModuleLaunchKernel(m->list[dev], (unsigned)(B * s.n_qt), 1, 1, 256, 1, 1, 0, st,
                               targs, nullptr) != hipSuccess)) {
      (void)hipGetLastError();
      return fail(ATTN_ERR_LAUNCH, "mask table kernel launch failed");
    }
    a.cls = t.cls;
    a.cnt = t.cnt;
    a.list = t.list;
    a.wfull = t.wfull;
  }
  void *const *ev = params->timing_events;
  if (ev && hipEventRecord((hipEvent_t)ev[0], st) != hipSuccess)
    return fail(ATTN_ERR_LAUNCH, "timing event record failed");
  void *fargs[] = {&a};
  // d = 256: two workgroups per (q-tile, head), one per half of the columns of O
  if (hipModuleLaunchKernel(m->fwd[dev][params->o_dtype == ATTN_O_F32 ? 1 : 0],
                            (unsigned)(s.n_qt * B * H), d > 128 ? 2 : 1, 1, 512, 1, 1, 0, st,
                            fargs, nullptr) != hipSuccess) {
    (void)hipGetLastError();
    return fail(ATTN_ERR_LAUNCH, "forward kernel launch failed");
  }
  if (ev && hipEventRecord((hipEvent_t)ev[1], st) != hipSuccess)
    return fail(ATTN_ERR_LAUNCH, "timing event record failed");
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd_mod(const attn_mod *m, const void *q, const void *k, const void *v, void *o,
                 float *lse, int B, int H, int N, float scale, const float *mod_params,
                 const attn_params *params, void *stream) {
  return fwd_mod(m, q, k, v, o, lse, B, H, N, scale, mod_params, params, stream, true);
}

int attn_fwd_mod_cached(const attn_mod *m, const void *q, const void *k, const void *v, void *o,
                        float *lse, int B, int H, int N, float scale, const float *mod_params,
                        const attn_params *params, void *stream) {
  return fwd_mod(m, q, k, v, o, lse, B, H, N, scale, mod_params, params, stream, false);
}

}  // extern "C"
