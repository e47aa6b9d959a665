// Host layer of libfibatt: argument validation, the Wythoff helpers, the
// per-head window interpolation, the offset table and the workspace sizes.
// Plain C++17 (no HIP): the library builds it with the host compiler, and a
// CPU test builds it again with AddressSanitizer and UndefinedBehaviorSanitizer.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "validate.h"

namespace fibatt {
namespace host {
namespace {

thread_local std::string g_error;

using u128 = unsigned __int128;

// floor(sqrt(x)), exact for every 128-bit x below 2^126 (the squares it is
// asked about stay far below that).
u128 isqrt128(u128 x) {
  u128 r = static_cast<u128>(std::sqrt(static_cast<long double>(x)));
  while (r * r > x) --r;
  while ((r + 1) * (r + 1) <= x) ++r;
  return r;
}

// floor(n * phi) = floor((n + sqrt(5 n^2)) / 2): sqrt(5 n^2) is irrational
// for n >= 1, so flooring it first does not change the result.  Exact for
// n < 2^62 (5 n^2 < 2^127).
uint64_t floor_n_phi(uint64_t n) {
  const u128 s = isqrt128(static_cast<u128>(5) * n * n);
  return static_cast<uint64_t>((static_cast<u128>(n) + s) / 2);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_heads(int32_t H, int32_t N, const int32_t* a, const int32_t* b, const int32_t* w) {
  if (!a || !b || !w) return fail(FIBATT_E_INVAL, "a, b and w must be non-NULL host arrays");
  for (int h = 0; h < H; ++h) {
    if (a[h] < 0) return fail(FIBATT_E_INVAL, "a[%d] = %d must be >= 0", h, a[h]);
    if (b[h] < 1) return fail(FIBATT_E_INVAL, "b[%d] = %d must be >= 1", h, b[h]);
    if (w[h] < 1 || w[h] > N)
      return fail(FIBATT_E_INVAL, "w[%d] = %d must lie in [1, N = %d]", h, w[h], N);
  }
  return FIBATT_OK;
}

// Shape and type checks shared by both descriptor kinds; fills p's sizes.
int check_shape(int32_t B, int32_t H, int32_t N, int32_t d_h, int32_t dtype, Problem* p) {
  if (B < 1 || H < 1 || N < 1)
    return fail(FIBATT_E_INVAL, "B, H, N must be >= 1 (got %d, %d, %d)", B, H, N);
  if (d_h != 64 && d_h != 128)
    return fail(FIBATT_E_UNSUPPORTED, "d_h = %d: supported head widths are 64 and 128", d_h);
  if (dtype != FIBATT_F32 && dtype != FIBATT_BF16)
    return fail(FIBATT_E_UNSUPPORTED, "dtype %d: supported are FIBATT_F32 and FIBATT_BF16",
                dtype);
  if (H > FIBATT_MAX_HEADS)
    return fail(FIBATT_E_UNSUPPORTED, "H = %d exceeds FIBATT_MAX_HEADS = %d", H,
                FIBATT_MAX_HEADS);
  const int64_t slabs = static_cast<int64_t>(B) * H;
  // Kernel grids are 1-D with at most 2^31 - 1 workgroups (the smallest row
  // tile is 32 rows, and the streaming backward launches two tiles per
  // tile); element offsets are computed in 64-bit.
  const int64_t tiles = (static_cast<int64_t>(N) + 31) / 32;
  if (slabs > 0x7fffffffll / (2 * tiles))
    return fail(FIBATT_E_UNSUPPORTED, "B*H*N too large for one launch");
  p->B = B;
  p->H = H;
  p->N = N;
  p->D = d_h;
  p->dtype = dtype == FIBATT_BF16 ? DType::kBF16 : DType::kF32;
  p->dense_layouts();
  return FIBATT_OK;
}

// Validates one tensor's layout (strides in elements of esize bytes).  A
// tensor the call writes must give every (batch, head) slab rows of its own:
// a zero batch stride with B > 1, or a zero head stride with H > 1, would
// have several slabs store to the same rows.
int check_layout(const fibatt_layout& l, const char* name, const Problem& p, int esize,
                 bool written, Layout* out) {
  if (l.sb < 0 || l.sh < 0 || l.sn < 0)
    return fail(FIBATT_E_INVAL, "layout of %s: strides must be >= 0", name);
  if (l.sn < p.D)
    return fail(FIBATT_E_INVAL, "layout of %s: sn = %lld must be >= d_h = %d", name,
                static_cast<long long>(l.sn), p.D);
  const int64_t unit = 16 / esize;
  if (l.sb % unit || l.sh % unit || l.sn % unit)
    return fail(FIBATT_E_INVAL, "layout of %s: strides must be multiples of %lld elements", name,
                static_cast<long long>(unit));
  // Largest element offset, with every term kept below 2^62.
  const int64_t lim = int64_t{1} << 62;
  const int64_t n[3] = {p.B - 1, p.H - 1, p.N - 1};
  const int64_t st[3] = {l.sb, l.sh, l.sn};
  int64_t end = p.D;
  for (int i = 0; i < 3; ++i) {
    if (st[i] && n[i] > (lim - end) / st[i])
      return fail(FIBATT_E_INVAL, "layout of %s: offsets exceed 2^62 elements", name);
    end += n[i] * st[i];
  }
  if (written && ((l.sb == 0 && p.B > 1) || (l.sh == 0 && p.H > 1)))
    return fail(FIBATT_E_INVAL,
                "layout of %s: an output needs non-zero batch and head strides when B or H > 1 "
                "(broadcast strides are for inputs only)",
                name);
  *out = Layout{l.sb, l.sh, l.sn};
  return FIBATT_OK;
}

bool same_layout(const Layout& x, const Layout& y) {
  return x.sb == y.sb && x.sh == y.sh && x.sn == y.sn;
}

}  // namespace

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return FIBATT_OK;
}

int check_desc(const fibatt_desc* d, Problem* p) {
  if (!d) return fail(FIBATT_E_INVAL, "desc is NULL");
  int rc = check_shape(d->B, d->H, d->N, d->d_h, d->dtype, p);
  if (rc) return rc;
  rc = check_heads(d->H, d->N, d->a, d->b, d->w);
  if (rc) return rc;
  p->heads.table = nullptr;
  p->host_table = nullptr;
  for (int h = 0; h < d->H; ++h) {
    p->heads.a[h] = d->a[h];
    p->heads.b[h] = d->b[h];
    p->heads.lim[h] = (d->w[h] < d->N - 1) ? d->w[h] : d->N - 1;
  }
  return FIBATT_OK;
}

int check_table_desc(const fibatt_table_desc* d, Problem* p) {
  if (!d) return fail(FIBATT_E_INVAL, "desc is NULL");
  int rc = check_shape(d->B, d->H, d->N, d->d_h, d->dtype, p);
  if (rc) return rc;
  if (d->cls != 0 && d->cls != 1) return fail(FIBATT_E_INVAL, "cls must be 0 or 1");
  if (!d->head_ptr) return fail(FIBATT_E_INVAL, "head_ptr is NULL");
  if (d->head_ptr[0] != 0) return fail(FIBATT_E_INVAL, "head_ptr[0] must be 0");
  for (int h = 0; h < d->H; ++h) {
    if (d->head_ptr[h + 1] < d->head_ptr[h])
      return fail(FIBATT_E_INVAL, "head_ptr must be non-decreasing (head %d)", h);
    const int64_t n = static_cast<int64_t>(d->head_ptr[h + 1]) - d->head_ptr[h];
    if (n > kMaxOffsets)
      return fail(FIBATT_E_UNSUPPORTED, "head %d has %lld distances; at most %d are supported",
                  h, static_cast<long long>(n), kMaxOffsets);
  }
  const int32_t total = d->head_ptr[d->H];
  if (total > 0 && (!d->offs || !d->offs_device))
    return fail(FIBATT_E_INVAL, "offs and offs_device must be non-NULL");
  if (total > 0 && (reinterpret_cast<uintptr_t>(d->offs_device) & 3u))
    return fail(FIBATT_E_INVAL, "offs_device is not 4-byte aligned");
  for (int h = 0; h < d->H; ++h) {
    for (int32_t i = d->head_ptr[h]; i < d->head_ptr[h + 1]; ++i) {
      const int32_t f = d->offs[i];
      if (f < 0 || f >= d->N)
        return fail(FIBATT_E_INVAL, "head %d: distance %d outside [0, N - 1 = %d]", h, f,
                    d->N - 1);
      if (i > d->head_ptr[h] && f <= d->offs[i - 1])
        return fail(FIBATT_E_INVAL, "head %d: distances must be strictly ascending", h);
    }
    p->heads.a[h] = d->head_ptr[h];
    p->heads.b[h] = d->head_ptr[h + 1] - d->head_ptr[h];
    p->heads.lim[h] = d->N - 1;
  }
  p->heads.table = d->offs_device;
  p->host_table = d->offs;
  p->cls = d->cls != 0;
  return FIBATT_OK;
}

int check_ptr(const void* ptr, const char* name) {
  if (!ptr) return fail(FIBATT_E_INVAL, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(FIBATT_E_INVAL, "%s is not 16-byte aligned", name);
  return FIBATT_OK;
}

int check_layouts(const fibatt_layouts* ls, bool bwd, Problem* p) {
  if (!ls) return fail(FIBATT_E_INVAL, "layouts is NULL");
  const int es = p->dtype == DType::kBF16 ? 2 : 4;
  int rc;
  if ((rc = check_layout(ls->q, "q", *p, es, false, &p->lq)) ||
      (rc = check_layout(ls->k, "k", *p, es, false, &p->lk)) ||
      (rc = check_layout(ls->v, "v", *p, es, false, &p->lv)))
    return rc;
  if (bwd) {
    if ((rc = check_layout(ls->dout, "dout", *p, es, false, &p->ldo)) ||
        (rc = check_layout(ls->dq, "dq", *p, 4, true, &p->ldq)) ||
        (rc = check_layout(ls->dk, "dk", *p, 4, true, &p->ldk)) ||
        (rc = check_layout(ls->dv, "dv", *p, 4, true, &p->ldv)))
      return rc;
  } else if ((rc = check_layout(ls->o, "o", *p, es, true, &p->lo))) {
    return rc;
  }
  const Layout d{static_cast<int64_t>(p->H) * p->N * p->D, static_cast<int64_t>(p->N) * p->D,
                 p->D};
  const Layout* used[] = {&p->lq, &p->lk, &p->lv, bwd ? &p->ldo : &p->lo,
                          &p->ldq, &p->ldk, &p->ldv};
  const int n_used = bwd ? 7 : 4;
  p->strided = false;
  for (int i = 0; i < n_used; ++i) p->strided |= !same_layout(*used[i], d);
  return FIBATT_OK;
}

Path path_from_env() {
  const char* s = std::getenv("FIBATT_PATH");
  if (!s) return Path::kAuto;
  if (std::string(s) == "slab") return Path::kSlab;
  if (std::string(s) == "stream") return Path::kStream;
  return Path::kAuto;
}

}  // namespace host
}  // namespace fibatt

using fibatt::host::fail;
using fibatt::host::ok;

extern "C" {

int fibatt_wythoff(int32_t i, int32_t* a, int32_t* b) {
  if (!a || !b) return fail(FIBATT_E_INVAL, "output pointers must be non-NULL");
  if (i < 1) return fail(FIBATT_E_INVAL, "Wythoff rows are numbered from 1 (got %d)", i);
  const uint64_t p = fibatt::host::floor_n_phi(static_cast<uint64_t>(i));
  const uint64_t av = fibatt::host::floor_n_phi(p);
  const uint64_t bv = av + p;
  if (bv > 0x7fffffffull) return fail(FIBATT_E_RANGE, "row %d does not fit int32", i);
  *a = static_cast<int32_t>(av);
  *b = static_cast<int32_t>(bv);
  return ok();
}

// The modified pair is the row's recurrence taken two steps back, which for
// the Wythoff array is the closed form (i - 1, floor(i phi)): the two columns
// that precede the row's first entry in the extended array.
int fibatt_wythoff_modified(int32_t i, int32_t* a, int32_t* b) {
  if (!a || !b) return fail(FIBATT_E_INVAL, "output pointers must be non-NULL");
  if (i < 1) return fail(FIBATT_E_INVAL, "Wythoff rows are numbered from 1 (got %d)", i);
  const uint64_t p = fibatt::host::floor_n_phi(static_cast<uint64_t>(i));
  if (p > 0x7fffffffull) return fail(FIBATT_E_RANGE, "row %d does not fit int32", i);
  *a = i - 1;
  *b = static_cast<int32_t>(p);
  return ok();
}

int fibatt_windows(int32_t H, int32_t w_min, int32_t w_max, int32_t* w) {
  if (H < 1 || !w) return fail(FIBATT_E_INVAL, "need H >= 1 and a non-NULL w");
  if (w_min < 1 || w_max < w_min)
    return fail(FIBATT_E_INVAL, "need 1 <= w_min <= w_max (got %d, %d)", w_min, w_max);
  if (H == 1) {
    w[0] = w_max;
    return ok();
  }
  for (int32_t i = 1; i <= H; ++i)
    w[i - 1] = w_min + static_cast<int32_t>(static_cast<int64_t>(w_max - w_min) * (i - 1) / (H - 1));
  return ok();
}

int fibatt_offsets(int32_t H, int32_t N, const int32_t* a, const int32_t* b, const int32_t* w,
                   int32_t* head_ptr, int32_t* offs, int32_t offs_cap) {
  if (H < 1 || N < 1) return fail(FIBATT_E_INVAL, "H and N must be >= 1 (got %d, %d)", H, N);
  if (!head_ptr) return fail(FIBATT_E_INVAL, "head_ptr is NULL");
  if (offs_cap < 0 || (offs_cap > 0 && !offs))
    return fail(FIBATT_E_INVAL, "offs must be non-NULL when offs_cap > 0");
  int rc = fibatt::host::check_heads(H, N, a, b, w);
  if (rc) return rc;
  int32_t tmp[fibatt::kMaxOffsets];
  int64_t total = 0;
  head_ptr[0] = 0;
  for (int h = 0; h < H; ++h) {
    const int64_t lim = w[h] < N - 1 ? w[h] : N - 1;
    const int n = fibatt::fib_offsets_gen(a[h], b[h], lim, tmp, fibatt::kMaxOffsets);
    if (total + n > 0x7fffffffll) return fail(FIBATT_E_RANGE, "offset table exceeds int32");
    total += n;
    head_ptr[h + 1] = static_cast<int32_t>(total);
  }
  if (total > offs_cap)
    return fail(FIBATT_E_RANGE, "offs needs %lld entries, capacity %d", (long long)total,
                offs_cap);
  for (int h = 0; h < H; ++h) {
    const int64_t lim = w[h] < N - 1 ? w[h] : N - 1;
    fibatt::fib_offsets_gen(a[h], b[h], lim, offs + head_ptr[h], fibatt::kMaxOffsets);
  }
  return ok();
}

int64_t fibatt_bwd_workspace_floats(const fibatt_desc* desc) {
  fibatt::Problem p;
  if (fibatt::host::check_desc(desc, &p)) return -1;
  ok();
  return static_cast<int64_t>(p.B) * p.H * p.N;
}

int64_t fibatt_fwd_cls_workspace_floats(const fibatt_desc* desc) {
  fibatt::Problem p;
  if (fibatt::host::check_desc(desc, &p)) return -1;
  ok();
  return fibatt::fwd_cls_workspace_floats(p);
}

int64_t fibatt_bwd_cls_workspace_floats(const fibatt_desc* desc) {
  fibatt::Problem p;
  if (fibatt::host::check_desc(desc, &p)) return -1;
  ok();
  return fibatt::bwd_cls_workspace_floats(p);
}

int64_t fibatt_fwd_table_workspace_floats(const fibatt_table_desc* desc) {
  fibatt::Problem p;
  if (fibatt::host::check_table_desc(desc, &p)) return -1;
  ok();
  return p.cls ? fibatt::fwd_cls_workspace_floats(p) : 0;
}

int64_t fibatt_bwd_table_workspace_floats(const fibatt_table_desc* desc) {
  fibatt::Problem p;
  if (fibatt::host::check_table_desc(desc, &p)) return -1;
  ok();
  return p.cls ? fibatt::bwd_cls_workspace_floats(p) : static_cast<int64_t>(p.B) * p.H * p.N;
}

const char* fibatt_last_error(void) { return fibatt::host::g_error.c_str(); }

}  // extern "C"
