// layout.cpp -- the Shape:Stride layout algebra (host only) and its C entry
// points.  Definitions follow "CuTe's layout algebra": a layout maps a
// coordinate to its inner product with the stride ("A layout: shape and
// stride"); coalesce preserves the function on one-dimensional coordinates
// ("Coalescing"); composition R = A o B has R(c) = A(B(c)) and B's shape
// ("Composition"); complement(A, M) lays out the indices of [0, M) that A
// misses so that (A, A*) covers each once, and logical_divide(A, B) =
// A o (B, complement(B, size A)) ("Complement and division"); local_tile and
// local_partition fix one mode of a zipped divide ("From tiles to threads").
#include "layout.hpp"

#include <algorithm>
#include <cctype>
#include <cstring>
#include <utility>

#include "../../include/thl.h"

namespace thl {

// ------------------------------------------------------------------ tuples

bool IntTuple::operator==(const IntTuple& o) const {
  if (leaf != o.leaf) return false;
  if (leaf) return value == o.value;
  return kids == o.kids;
}

static int64_t product(const IntTuple& t) {
  if (t.leaf) return t.value;
  int64_t p = 1;
  for (const auto& k : t.kids) p *= product(k);
  return p;
}

static void leaves(const IntTuple& t, std::vector<int64_t>* out) {
  if (t.leaf) {
    out->push_back(t.value);
    return;
  }
  for (const auto& k : t.kids) leaves(k, out);
}

static bool congruent(const IntTuple& a, const IntTuple& b) {
  if (a.leaf || b.leaf) return a.leaf == b.leaf;
  if (a.kids.size() != b.kids.size()) return false;
  for (size_t i = 0; i < a.kids.size(); ++i)
    if (!congruent(a.kids[i], b.kids[i])) return false;
  return true;
}

std::string str(const IntTuple& t) {
  if (t.leaf) return std::to_string(t.value);
  std::string s = "(";
  for (size_t i = 0; i < t.kids.size(); ++i) {
    if (i) s += ",";
    s += str(t.kids[i]);
  }
  return s + ")";
}

namespace {
struct Parser {
  const std::string& s;
  size_t pos = 0;
  explicit Parser(const std::string& text) : s(text) {}
  void skip() {
    while (pos < s.size() && (std::isspace(static_cast<unsigned char>(s[pos])) || s[pos] == '_')) ++pos;
  }
  [[noreturn]] void fail(const char* what) {
    throw LayoutError(LayoutError::kParse, std::string(what) + " at offset " + std::to_string(pos) + " in '" + s + "'");
  }
  IntTuple tuple() {
    skip();
    if (pos < s.size() && s[pos] == '(') {
      ++pos;
      std::vector<IntTuple> kids;
      for (;;) {
        kids.push_back(tuple());
        skip();
        if (pos < s.size() && s[pos] == ',') {
          ++pos;
          continue;
        }
        if (pos < s.size() && s[pos] == ')') {
          ++pos;
          break;
        }
        fail("expected ',' or ')'");
      }
      return IntTuple::node(std::move(kids));
    }
    bool neg = false;
    if (pos < s.size() && s[pos] == '-') {
      neg = true;
      ++pos;
    }
    if (pos >= s.size() || !std::isdigit(static_cast<unsigned char>(s[pos]))) fail("expected an integer");
    int64_t v = 0;
    while (pos < s.size() && std::isdigit(static_cast<unsigned char>(s[pos]))) {
      v = v * 10 + (s[pos] - '0');
      ++pos;
    }
    return IntTuple::of(neg ? -v : v);
  }
  bool at_end() {
    skip();
    return pos == s.size();
  }
};
}  // namespace

IntTuple parse_tuple(const std::string& text) {
  Parser p(text);
  IntTuple t = p.tuple();
  if (!p.at_end()) p.fail("trailing text");
  return t;
}

// "shape:stride", or a bare shape meaning the compact column-major layout.
Layout parse_layout(const std::string& text) {
  size_t colon = text.find(':');
  if (colon == std::string::npos) return Layout::compact(parse_tuple(text));
  return Layout(parse_tuple(text.substr(0, colon)), parse_tuple(text.substr(colon + 1)));
}

// ------------------------------------------------------------------ layout

Layout::Layout(IntTuple s, IntTuple d) : shape(std::move(s)), stride(std::move(d)) {
  if (!congruent(shape, stride)) throw LayoutError(LayoutError::kCongruence, "shape and stride differ in structure");
  std::vector<int64_t> sh;
  leaves(shape, &sh);
  for (int64_t v : sh)
    if (v < 0) throw LayoutError(LayoutError::kRange, "negative extent");
}

// Column-major: each leaf's stride is the product of the extents before it.
Layout Layout::compact(const IntTuple& shape) {
  int64_t running = 1;
  struct Walk {
    int64_t& run;
    IntTuple go(const IntTuple& s) {
      if (s.leaf) {
        IntTuple d = IntTuple::of(run);
        run *= s.value;
        return d;
      }
      std::vector<IntTuple> k;
      for (const auto& c : s.kids) k.push_back(go(c));
      return IntTuple::node(std::move(k));
    }
  } w{running};
  IntTuple d = w.go(shape);
  return Layout(shape, d);
}

int64_t Layout::size() const { return product(shape); }

// Split an integer coordinate over a (sub)shape, mode 0 fastest; the last
// mode takes whatever is left.
static int64_t index_of(int64_t c, const IntTuple& s, const IntTuple& d) {
  if (s.leaf) return c * d.value;
  int64_t idx = 0;
  const size_t n = s.kids.size();
  for (size_t i = 0; i + 1 < n; ++i) {
    const int64_t ext = product(s.kids[i]);
    idx += index_of(ext ? c % ext : 0, s.kids[i], d.kids[i]);
    c = ext ? c / ext : 0;
  }
  return idx + index_of(c, s.kids[n - 1], d.kids[n - 1]);
}

static int64_t index_of(const IntTuple& c, const IntTuple& s, const IntTuple& d) {
  if (c.leaf) return index_of(c.value, s, d);
  if (s.leaf || c.kids.size() != s.kids.size())
    throw LayoutError(LayoutError::kCongruence, "coordinate does not match the shape");
  int64_t idx = 0;
  for (size_t i = 0; i < c.kids.size(); ++i) idx += index_of(c.kids[i], s.kids[i], d.kids[i]);
  return idx;
}

int64_t Layout::operator()(int64_t crd) const { return index_of(crd, shape, stride); }
int64_t Layout::operator()(const IntTuple& crd) const { return index_of(crd, shape, stride); }

int64_t Layout::cosize() const {
  const int64_t n = size();
  return n == 0 ? 0 : (*this)(n - 1) + 1;
}

Layout Layout::mode(size_t i) const {
  if (shape.leaf) {
    if (i != 0) throw LayoutError(LayoutError::kRange, "mode index out of range");
    return *this;
  }
  if (i >= shape.kids.size()) throw LayoutError(LayoutError::kRange, "mode index out of range");
  return Layout(shape.kids[i], stride.kids[i]);
}

std::string Layout::str() const { return thl::str(shape) + ":" + thl::str(stride); }

int64_t SwizzledLayout::swizzle(int b, int m, int s, int64_t x) {
  const int64_t mask = (int64_t(1) << b) - 1;
  return x ^ (((x >> (m + s)) & mask) << m);
}

int64_t SwizzledLayout::operator()(int64_t crd) const { return swizzle(b, m, s, inner(crd)); }

// ------------------------------------------------------------------ algebra

Layout make_layout(const std::vector<Layout>& modes) {
  std::vector<IntTuple> s, d;
  for (const auto& l : modes) {
    s.push_back(l.shape);
    d.push_back(l.stride);
  }
  return Layout(IntTuple::node(std::move(s)), IntTuple::node(std::move(d)));
}

// Build a layout from flat (extent, stride) lists: one mode stays a leaf.
static Layout from_flat(const std::vector<int64_t>& s, const std::vector<int64_t>& d) {
  if (s.size() == 1) return Layout(IntTuple::of(s[0]), IntTuple::of(d[0]));
  std::vector<IntTuple> ks, kd;
  for (size_t i = 0; i < s.size(); ++i) {
    ks.push_back(IntTuple::of(s[i]));
    kd.push_back(IntTuple::of(d[i]));
  }
  return Layout(IntTuple::node(std::move(ks)), IntTuple::node(std::move(kd)));
}

Layout coalesce(const Layout& a) {
  std::vector<int64_t> s, d;
  leaves(a.shape, &s);
  leaves(a.stride, &d);
  std::vector<int64_t> rs, rd;
  for (size_t i = 0; i < s.size(); ++i) {
    if (s[i] == 1) continue;  // a size-1 mode contributes nothing
    if (!rs.empty() && rs.back() * rd.back() == d[i]) {
      rs.back() *= s[i];  // this mode continues exactly where the previous ended
    } else {
      rs.push_back(s[i]);
      rd.push_back(d[i]);
    }
  }
  if (rs.empty()) return Layout(IntTuple::of(1), IntTuple::of(0));
  return from_flat(rs, rd);
}

// A o (n:d): the layout of the n one-dimensional coordinates 0, d, 2d, ... of
// A.  Walk A's coalesced modes: a mode whose extent divides the remaining
// step is passed over whole; otherwise the step must divide the extent, the
// mode supplies extent/step elements at stride step*stride, and when it
// cannot supply all that remain their count must be a multiple of what it
// supplies.  A's last mode extends without bound.
static Layout compose_mode(const Layout& a, int64_t n, int64_t d) {
  if (n == 1) return Layout(IntTuple::of(1), IntTuple::of(0));
  if (d == 0) return Layout(IntTuple::of(n), IntTuple::of(0));
  Layout ca = coalesce(a);
  std::vector<int64_t> s, t;
  leaves(ca.shape, &s);
  leaves(ca.stride, &t);
  std::vector<int64_t> rs, rd;
  int64_t remaining = n, step = d;
  for (size_t i = 0; i + 1 < s.size() && remaining > 1; ++i) {
    if (step % s[i] == 0) {
      step /= s[i];
      continue;
    }
    if (s[i] % step != 0)
      throw LayoutError(LayoutError::kStrideDivisibility, "stride divisibility fails: composition undefined");
    const int64_t avail = s[i] / step;
    if (remaining <= avail) {
      rs.push_back(remaining);
      rd.push_back(step * t[i]);
      remaining = 1;
      break;
    }
    if (remaining % avail != 0)
      throw LayoutError(LayoutError::kShapeDivisibility, "shape divisibility fails: composition undefined");
    rs.push_back(avail);
    rd.push_back(step * t[i]);
    remaining /= avail;
    step = 1;
  }
  if (remaining > 1 || rs.empty()) {
    rs.push_back(remaining);
    rd.push_back(step * t.back());
  }
  return from_flat(rs, rd);
}

// Replace every leaf (n, d) of B by A o (n:d), keeping B's nesting.
static void compose_tree(const Layout& a, const IntTuple& bs, const IntTuple& bd, IntTuple* rs, IntTuple* rd) {
  if (bs.leaf) {
    Layout r = compose_mode(a, bs.value, bd.value);
    *rs = r.shape;
    *rd = r.stride;
    return;
  }
  std::vector<IntTuple> ks(bs.kids.size()), kd(bs.kids.size());
  for (size_t i = 0; i < bs.kids.size(); ++i) compose_tree(a, bs.kids[i], bd.kids[i], &ks[i], &kd[i]);
  *rs = IntTuple::node(std::move(ks));
  *rd = IntTuple::node(std::move(kd));
}

Layout composition(const Layout& a, const Layout& b) {
  IntTuple rs, rd;
  compose_tree(a, b.shape, b.stride, &rs, &rd);
  return Layout(rs, rd);
}

Layout composition(const Layout& a, const std::vector<Layout>& tiler) {
  if (tiler.size() > a.rank()) throw LayoutError(LayoutError::kRange, "tiler has more modes than the layout");
  std::vector<Layout> modes;
  for (size_t i = 0; i < a.rank(); ++i) modes.push_back(i < tiler.size() ? composition(a.mode(i), tiler[i]) : a.mode(i));
  return make_layout(modes);
}

// Fill the gaps of A inside [0, cotarget): visit A's modes by increasing
// stride; each gap before a mode becomes a mode whose stride is the span
// covered so far, and a last mode repeats the whole up to the cotarget.
Layout complement(const Layout& a, int64_t cotarget) {
  std::vector<int64_t> s, d;
  leaves(a.shape, &s);
  leaves(a.stride, &d);
  std::vector<std::pair<int64_t, int64_t>> modes;  // (stride, extent)
  for (size_t i = 0; i < s.size(); ++i)
    if (s[i] != 1 && d[i] != 0) modes.emplace_back(d[i], s[i]);
  std::sort(modes.begin(), modes.end());
  std::vector<int64_t> rs, rd;
  int64_t covered = 1;
  for (const auto& m : modes) {
    if (m.first % covered != 0) throw LayoutError(LayoutError::kOverlap, "modes overlap: complement undefined");
    rs.push_back(m.first / covered);
    rd.push_back(covered);
    covered = m.first * m.second;
  }
  rs.push_back((cotarget + covered - 1) / covered);
  rd.push_back(covered);
  return coalesce(from_flat(rs, rd));
}

Layout logical_divide(const Layout& a, const Layout& b) {
  return composition(a, make_layout({b, complement(b, a.size())}));
}

Layout logical_divide(const Layout& a, const std::vector<Layout>& tiler) {
  if (tiler.size() > a.rank()) throw LayoutError(LayoutError::kRange, "tiler has more modes than the layout");
  std::vector<Layout> modes;
  for (size_t i = 0; i < a.rank(); ++i) modes.push_back(i < tiler.size() ? logical_divide(a.mode(i), tiler[i]) : a.mode(i));
  return make_layout(modes);
}

static void split_divide(const Layout& a, const std::vector<Layout>& tiler, std::vector<Layout>* inner,
                         std::vector<Layout>* outer) {
  Layout d = logical_divide(a, tiler);
  for (size_t i = 0; i < tiler.size(); ++i) {
    inner->push_back(d.mode(i).mode(0));
    outer->push_back(d.mode(i).mode(1));
  }
  for (size_t i = tiler.size(); i < a.rank(); ++i) outer->push_back(d.mode(i));
}

Layout zipped_divide(const Layout& a, const std::vector<Layout>& tiler) {
  std::vector<Layout> in, out;
  split_divide(a, tiler, &in, &out);
  return make_layout({make_layout(in), make_layout(out)});
}

Layout tiled_divide(const Layout& a, const std::vector<Layout>& tiler) {
  std::vector<Layout> in, out;
  split_divide(a, tiler, &in, &out);
  std::vector<Layout> modes{make_layout(in)};
  modes.insert(modes.end(), out.begin(), out.end());
  return make_layout(modes);
}

Layout flat_divide(const Layout& a, const std::vector<Layout>& tiler) {
  std::vector<Layout> in, out;
  split_divide(a, tiler, &in, &out);
  in.insert(in.end(), out.begin(), out.end());
  return make_layout(in);
}

Layout local_tile(const Layout& a, const std::vector<Layout>& tiler, int64_t tile, int64_t* offset) {
  Layout z = zipped_divide(a, tiler);
  Layout which = z.mode(1);
  if (tile < 0 || tile >= which.size()) throw LayoutError(LayoutError::kRange, "tile index out of range");
  *offset = which(tile);
  return z.mode(0);
}

Layout local_partition(const Layout& a, const Layout& threads, int64_t tid, int64_t* offset) {
  std::vector<Layout> tiler;
  for (size_t i = 0; i < threads.rank(); ++i) tiler.push_back(Layout::compact(threads.mode(i).shape));
  Layout z = zipped_divide(a, tiler);
  const int64_t nthr = threads.size();
  int64_t pos = -1;
  for (int64_t p = 0; p < nthr; ++p)
    if (threads(p) == tid) {
      pos = p;
      break;
    }
  if (pos < 0) throw LayoutError(LayoutError::kRange, "thread id not in the thread layout");
  *offset = z.mode(0)(pos);
  return z.mode(1);
}

}  // namespace thl

// ------------------------------------------------------------------ C ABI

namespace {

int status_of(const thl::LayoutError& e) {
  switch (e.kind) {
    case thl::LayoutError::kShapeDivisibility:
    case thl::LayoutError::kStrideDivisibility:
    case thl::LayoutError::kOverlap:
      return THL_ERR_UNDEFINED;
    default:
      return THL_ERR_INVALID;
  }
}

int put(const std::string& s, char* out, size_t cap) {
  if (!out || cap < s.size() + 1) return THL_ERR_INVALID;
  std::memcpy(out, s.c_str(), s.size() + 1);
  return THL_OK;
}

std::vector<thl::Layout> parse_tiler(const char* text) {
  std::vector<thl::Layout> t;
  std::string s(text);
  size_t start = 0;
  for (;;) {
    size_t semi = s.find(';', start);
    t.push_back(thl::parse_layout(s.substr(start, semi == std::string::npos ? std::string::npos : semi - start)));
    if (semi == std::string::npos) break;
    start = semi + 1;
  }
  return t;
}

template <class F>
int guarded(F&& f) {
  try {
    return f();
  } catch (const thl::LayoutError& e) {
    return status_of(e);
  } catch (...) {
    return THL_ERR_INVALID;
  }
}

}  // namespace

extern "C" {

int thl_layout_coalesce(const char* a, char* out, size_t cap) {
  if (!a) return THL_ERR_INVALID;
  return guarded([&] { return put(thl::coalesce(thl::parse_layout(a)).str(), out, cap); });
}

int thl_layout_composition(const char* a, const char* b, char* out, size_t cap) {
  if (!a || !b) return THL_ERR_INVALID;
  return guarded([&] {
    thl::Layout la = thl::parse_layout(a);
    if (std::strchr(b, ';')) return put(thl::composition(la, parse_tiler(b)).str(), out, cap);
    return put(thl::composition(la, thl::parse_layout(b)).str(), out, cap);
  });
}

int thl_layout_complement(const char* a, int64_t cotarget, char* out, size_t cap) {
  if (!a || cotarget < 0) return THL_ERR_INVALID;
  return guarded([&] { return put(thl::complement(thl::parse_layout(a), cotarget).str(), out, cap); });
}

int thl_layout_logical_divide(const char* a, const char* tiler, char* out, size_t cap) {
  if (!a || !tiler) return THL_ERR_INVALID;
  return guarded([&] {
    thl::Layout la = thl::parse_layout(a);
    if (std::strchr(tiler, ';')) return put(thl::logical_divide(la, parse_tiler(tiler)).str(), out, cap);
    return put(thl::logical_divide(la, thl::parse_layout(tiler)).str(), out, cap);
  });
}

int thl_layout_zipped_divide(const char* a, const char* tiler, char* out, size_t cap) {
  if (!a || !tiler) return THL_ERR_INVALID;
  return guarded([&] { return put(thl::zipped_divide(thl::parse_layout(a), parse_tiler(tiler)).str(), out, cap); });
}

int thl_layout_tiled_divide(const char* a, const char* tiler, char* out, size_t cap) {
  if (!a || !tiler) return THL_ERR_INVALID;
  return guarded([&] { return put(thl::tiled_divide(thl::parse_layout(a), parse_tiler(tiler)).str(), out, cap); });
}

int thl_layout_flat_divide(const char* a, const char* tiler, char* out, size_t cap) {
  if (!a || !tiler) return THL_ERR_INVALID;
  return guarded([&] { return put(thl::flat_divide(thl::parse_layout(a), parse_tiler(tiler)).str(), out, cap); });
}

int thl_layout_local_tile(const char* a, const char* tiler, int64_t tile, int64_t* offset, char* out, size_t cap) {
  if (!a || !tiler || !offset) return THL_ERR_INVALID;
  return guarded([&] {
    return put(thl::local_tile(thl::parse_layout(a), parse_tiler(tiler), tile, offset).str(), out, cap);
  });
}

int thl_layout_local_partition(const char* a, const char* threads, int64_t tid, int64_t* offset, char* out,
                               size_t cap) {
  if (!a || !threads || !offset) return THL_ERR_INVALID;
  return guarded([&] {
    return put(thl::local_partition(thl::parse_layout(a), thl::parse_layout(threads), tid, offset).str(), out, cap);
  });
}

int thl_layout_eval(const char* a, const int64_t* crd, int64_t n, int64_t* out) {
  if (!a || n < 0 || (n > 0 && (!crd || !out))) return THL_ERR_INVALID;
  return guarded([&] {
    thl::Layout l = thl::parse_layout(a);
    for (int64_t i = 0; i < n; ++i) out[i] = l(crd[i]);
    return THL_OK;
  });
}

int thl_layout_eval_coord(const char* a, const char* coord, int64_t* out) {
  if (!a || !coord || !out) return THL_ERR_INVALID;
  return guarded([&] {
    *out = thl::parse_layout(a)(thl::parse_tuple(coord));
    return THL_OK;
  });
}

int thl_layout_info(const char* a, int64_t* size, int64_t* cosize, int64_t* rank) {
  if (!a) return THL_ERR_INVALID;
  return guarded([&] {
    thl::Layout l = thl::parse_layout(a);
    if (size) *size = l.size();
    if (cosize) *cosize = l.cosize();
    if (rank) *rank = static_cast<int64_t>(l.rank());
    return THL_OK;
  });
}

int thl_layout_mode(const char* a, int64_t i, char* out, size_t cap) {
  if (!a || i < 0) return THL_ERR_INVALID;
  return guarded([&] { return put(thl::parse_layout(a).mode(static_cast<size_t>(i)).str(), out, cap); });
}

int thl_swizzle_eval(int b, int m, int s, const char* a, const int64_t* crd, int64_t n, int64_t* out) {
  if (!a || b < 0 || m < 0 || s < 0 || b + m + s > 62 || n < 0 || (n > 0 && (!crd || !out))) return THL_ERR_INVALID;
  return guarded([&] {
    thl::SwizzledLayout sl{b, m, s, thl::parse_layout(a)};
    for (int64_t i = 0; i < n; ++i) out[i] = sl(crd[i]);
    return THL_OK;
  });
}

}  // extern "C"
