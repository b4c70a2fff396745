// dispatch.cpp -- parser and lookup for the shape-keyed variant table.
#include "dispatch.hpp"

#include <cstdlib>
#include <sstream>

namespace lg {

namespace {

const char* kQuantNames[] = {"bf16", "fp16", "fp8_dynamic", "w8a8_int8", "block_fp8", "mxfp4"};

int quant_of(const std::string& s) {
  if (s == "*") return -1;
  for (int i = 0; i < 6; ++i)
    if (s == kQuantNames[i]) return i;
  return -2;
}

bool to_ll(const std::string& s, long long* v) {
  if (s == "*") { *v = -1; return true; }
  char* end = nullptr;
  long long x = std::strtoll(s.c_str(), &end, 10);
  if (!end || *end != '\0' || s.empty()) return false;
  *v = x;
  return true;
}

const char* reduce_name(int r) {
  switch (r) {
    case R_LASTWG: return "lastwg";
    case R_ATOMIC: return "atomic";
    case R_TWOPASS: return "twopass";
  }
  return "none";
}

}  // namespace

bool parse_variant(const std::string& spec, Variant* out, std::string* err) {
  std::istringstream is(spec);
  std::string kind;
  if (!(is >> kind)) { *err = "empty variant spec"; return false; }
  Variant v;
  if (kind == "tile") v.kind = V_TILE;
  else if (kind == "decode") v.kind = V_DECODE;
  else if (kind == "pp") v.kind = V_PP;
  else { *err = "unknown variant kind '" + kind + "'"; return false; }
  std::string kv;
  while (is >> kv) {
    size_t eq = kv.find('=');
    if (eq == std::string::npos) { *err = "expected key=value, got '" + kv + "'"; return false; }
    std::string k = kv.substr(0, eq), val = kv.substr(eq + 1);
    if (k == "reduce") {
      if (val == "lastwg") v.reduce = R_LASTWG;
      else if (val == "atomic") v.reduce = R_ATOMIC;
      else if (val == "twopass") v.reduce = R_TWOPASS;
      else if (val == "none") v.reduce = R_NONE;
      else { *err = "unknown reduce '" + val + "'"; return false; }
      continue;
    }
    long long x;
    if (!to_ll(val, &x) || x < 0) { *err = "bad value in '" + kv + "'"; return false; }
    int xi = (int)x;
    if (k == "bm") v.bm = xi;
    else if (k == "bn") v.bn = xi;
    else if (k == "wm") v.wm = xi;
    else if (k == "wn") v.wn = xi;
    else if (k == "group") v.group_m = xi;
    else if (k == "swap") v.swap = xi ? 1 : 0;
    else if (k == "split") v.split = xi;
    else if (k == "waves") v.waves = xi;
    else if (k == "unroll") v.unroll = xi;
    else if (k == "rows") v.rows = xi;
    else if (k == "dq") v.dq = xi ? 1 : 0;
    else if (k == "xs") {
      if (xi > 2) { *err = "xs must be 0, 1 or 2: " + spec; return false; }
      v.xs = xi;
    }
    else if (k == "sk") v.sk = xi;
    else { *err = "unknown key '" + k + "'"; return false; }
  }
  if (v.kind == V_TILE && !tile_supported(0, v.bm, v.bn, v.wm, v.wn)) {
    *err = "tile shape not compiled: " + spec;
    return false;
  }
  if (v.kind == V_TILE && v.sk > 8) {
    *err = "stream-K sk must be 0 (off) or 1..8 workgroups per CU: " + spec;
    return false;
  }
  if ((v.kind == V_PP || v.kind == V_TILE) && (v.split > 16 || (v.split & (v.split - 1)) != 0)) {
    *err = "tile / pp split must be 0 (auto) or a power of two <= 16: " + spec;
    return false;
  }
  if (v.kind == V_DECODE) {
    if (!decode_supported(v.swap, v.waves, v.unroll, v.rows)) {
      *err = "decode swap/waves/unroll/rows not compiled: " + spec;
      return false;
    }
    if (v.split > 256 || (v.split & (v.split - 1)) != 0) {
      *err = "split must be 0 (auto) or a power of two <= 256: " + spec;
      return false;
    }
  }
  *out = v;
  return true;
}

std::string format_variant(const Variant& v, int split) {
  std::ostringstream os;
  if (v.kind == V_TILE) {
    os << "tile bm=" << v.bm << " bn=" << v.bn << " wm=" << v.wm << " wn=" << v.wn
       << " group=" << v.group_m;
    if (v.sk > 0) os << " sk=" << v.sk;
    else if (split > 1) os << " split=" << split;
  } else if (v.kind == V_PP) {
    os << "pp split=" << split << " group=" << v.group_m;
  } else {
    os << "decode swap=" << v.swap << " split=" << split << " reduce=" << reduce_name(v.reduce)
       << " waves=" << v.waves << " unroll=" << v.unroll << " rows=" << v.rows;
    if (v.dq) os << " dq=1";
    if (v.xs) os << " xs=" << v.xs;
  }
  return os.str();
}

bool parse_table(const std::string& text, std::vector<TableEntry>* out, std::string* err) {
  std::istringstream is(text);
  std::string line;
  int lineno = 0;
  std::vector<TableEntry> t;
  while (std::getline(is, line)) {
    ++lineno;
    size_t hash = line.find('#');
    if (hash != std::string::npos) line = line.substr(0, hash);
    std::istringstream ls(line);
    std::string q, mlo, mhi, n, k;
    if (!(ls >> q)) continue;  // blank
    if (!(ls >> mlo >> mhi >> n >> k)) {
      *err = "line " + std::to_string(lineno) + ": expected <quant> <m_lo> <m_hi> <N> <K> <variant>";
      return false;
    }
    TableEntry e;
    e.quant = quant_of(q);
    if (e.quant == -2) { *err = "line " + std::to_string(lineno) + ": unknown quant '" + q + "'"; return false; }
    if (!to_ll(mlo, &e.m_lo) || e.m_lo < 0 || !to_ll(mhi, &e.m_hi) || !to_ll(n, &e.n) ||
        !to_ll(k, &e.k)) {
      *err = "line " + std::to_string(lineno) + ": bad number";
      return false;
    }
    std::string rest, tok;
    while (ls >> tok) rest += (rest.empty() ? "" : " ") + tok;
    std::string verr;
    if (!parse_variant(rest, &e.v, &verr)) {
      *err = "line " + std::to_string(lineno) + ": " + verr;
      return false;
    }
    if (e.v.kind == V_DECODE && (e.m_hi < 0 || e.m_hi > 32)) {
      *err = "line " + std::to_string(lineno) + ": decode entries must have m_hi <= 32";
      return false;
    }
    t.push_back(e);
  }
  *out = std::move(t);
  return true;
}

// Built-in table: the measured decode entries the offline sweep writes
// (table_mi355x.inc: exact (quant, N, K) shapes and token ranges), the
// measured prefill-shape entries, then the defaults: decode family for up to 32 tokens (swap-AB, K split among the
// waves of each workgroup), then tile sizes growing with M.
const char* builtin_table() {
  static const std::string text = std::string(
#include "table_mi355x.inc"
  ) + R"TABLE(
# prefill-shape entries (measured by the same sweep)
block_fp8      257  *    4096  12288  pp split=0 group=4
block_fp8      33   256  4096  12288  tile bm=64 bn=64 wm=2 wn=2 group=4
bf16           1025 *    4096  4096   pp group=4
bf16           33   256  256   512    tile bm=64 bn=64 wm=2 wn=2 group=4
mxfp4          33   1024 *     *      tile bm=64 bn=128 wm=1 wn=4 group=4
# defaults
*              1    32   *     *      decode swap=1 split=1 reduce=twopass waves=8 unroll=2
block_fp8      257  *    *     *      pp split=0 group=4
block_fp8      33   *    *     *      tile bm=128 bn=128 wm=2 wn=2 group=4
*              33   256  *     *      tile bm=64 bn=128 wm=1 wn=4 group=4
*              257  1024 *     *      tile bm=128 bn=128 wm=2 wn=4 group=4
bf16           1025 *    *     *      pp group=4
fp16           1025 *    *     *      pp group=4
w8a8_int8      1025 *    *     *      pp group=4
*              1025 *    *     *      tile bm=256 bn=256 wm=2 wn=4 group=4
)TABLE";
  return text.c_str();
}

bool lookup(const std::vector<TableEntry>& t, int quant, long long M, long long N, long long K,
            Variant* out) {
  for (const TableEntry& e : t) {
    if (e.quant >= 0 && e.quant != quant) continue;
    if (M < e.m_lo) continue;
    if (e.m_hi >= 0 && M > e.m_hi) continue;
    if (e.n >= 0 && e.n != N) continue;
    if (e.k >= 0 && e.k != K) continue;
    *out = e.v;
    return true;
  }
  return false;
}

}  // namespace lg
