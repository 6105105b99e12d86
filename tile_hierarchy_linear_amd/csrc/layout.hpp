// layout.hpp -- host-side Shape:Stride layout algebra.
//
// A layout is a pair of congruent nested integer tuples, shape and stride; it
// is the function from a coordinate to the inner product of that coordinate
// with the stride.  A one-dimensional coordinate is split colexicographically
// (mode 0 fastest) and the last mode is not reduced, so coordinates past the
// end extend along it.  Operations: coalesce, composition, complement,
// logical / zipped / tiled / flat divide, local_tile, local_partition, and an
// XOR swizzle composed on top of a layout.  ("CuTe's layout algebra", sections
// "A layout: shape and stride", "Coalescing", "Composition", "Complement and
// division", "From tiles to threads".)
//
// Everything here runs on the host with run-time integers and simplifies
// fully (coalesce merges as far as the function allows).  The GEMM kernels use
// closed-form index functions; tests check those against this module point by
// point.
#pragma once

#include <cstdint>
#include <stdexcept>
#include <string>
#include <vector>

namespace thl {

// A nested tuple of integers: a leaf holds one value, a node holds children.
struct IntTuple {
  bool leaf = true;
  int64_t value = 0;
  std::vector<IntTuple> kids;

  static IntTuple of(int64_t v) {
    IntTuple t;
    t.value = v;
    return t;
  }
  static IntTuple node(std::vector<IntTuple> k) {
    IntTuple t;
    t.leaf = false;
    t.kids = std::move(k);
    return t;
  }
  size_t rank() const { return leaf ? 1 : kids.size(); }
  bool operator==(const IntTuple& o) const;
};

// Raised for operations the algebra leaves undefined (a divisibility
// condition fails, modes overlap) and for malformed input.
struct LayoutError : std::runtime_error {
  enum Kind { kParse, kShapeDivisibility, kStrideDivisibility, kOverlap, kRange, kCongruence };
  Kind kind;
  LayoutError(Kind k, const std::string& what) : std::runtime_error(what), kind(k) {}
};

struct Layout {
  IntTuple shape, stride;

  Layout() = default;
  Layout(IntTuple s, IntTuple d);
  static Layout compact(const IntTuple& shape);  // column-major default stride

  int64_t size() const;
  int64_t cosize() const;  // largest index + 1 (for non-negative strides)
  size_t rank() const { return shape.rank(); }
  Layout mode(size_t i) const;
  int64_t operator()(int64_t crd) const;            // one-dimensional coordinate
  int64_t operator()(const IntTuple& crd) const;    // top-level or nested coordinate
  bool operator==(const Layout& o) const { return shape == o.shape && stride == o.stride; }
  std::string str() const;
};

// A layout whose index is passed through the XOR swizzle
//   s(x) = x ^ (((x >> (m + s)) & (2^b - 1)) << m).
struct SwizzledLayout {
  int b, m, s;
  Layout inner;
  int64_t operator()(int64_t crd) const;
  static int64_t swizzle(int b, int m, int s, int64_t x);
};

IntTuple parse_tuple(const std::string& text);
Layout parse_layout(const std::string& text);
std::string str(const IntTuple& t);

Layout make_layout(const std::vector<Layout>& modes);  // side by side
Layout coalesce(const Layout& a);
Layout composition(const Layout& a, const Layout& b);
Layout composition(const Layout& a, const std::vector<Layout>& tiler);  // mode by mode
Layout complement(const Layout& a, int64_t cotarget);
Layout logical_divide(const Layout& a, const Layout& b);
Layout logical_divide(const Layout& a, const std::vector<Layout>& tiler);
Layout zipped_divide(const Layout& a, const std::vector<Layout>& tiler);
Layout tiled_divide(const Layout& a, const std::vector<Layout>& tiler);
Layout flat_divide(const Layout& a, const std::vector<Layout>& tiler);

// The tile of `a` with tile index `tile` (a one-dimensional coordinate over
// the tile-index modes): returns its layout and the index offset of its origin.
Layout local_tile(const Layout& a, const std::vector<Layout>& tiler, int64_t tile, int64_t* offset);
// The values thread `tid` owns when `a` is divided by the shape of `threads`:
// the thread takes the within-tile position p with threads(p) == tid, and its
// values are the tile-index mode.  Returns that mode and the offset of p.
Layout local_partition(const Layout& a, const Layout& threads, int64_t tid, int64_t* offset);

}  // namespace thl
