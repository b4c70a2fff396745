// dispatch.hpp -- the shape-keyed variant table.
//
// One kernel family per regime, with the choices that matter per shape kept
// as table fields rather than separate code paths (the approach of
// "helion-vllm-linear-backend", section "Одно ядро вместо трёх вариантов":
// split_k as a power of two up to 256 and swap_ab as a boolean, picked per
// shape), and small token counts routed to the decode family (section
// "Гибридный диспатч": shapes up to 32 tokens take the tuned path).  The
// table is filled by the offline sweep; a built-in table is the default that
// tests and CI run on.
//
// Text format, one entry per line ('#' starts a comment):
//   <quant|*> <m_lo> <m_hi|*> <N|*> <K|*> <variant spec>
// where the variant spec is
//   tile   bm=<tokens> bn=<weight rows> wm=<waves> wn=<waves> [group=<g>]
//          [split=<0=auto|1..16>]   (K split across workgroups, two-pass)
//   pp     [split=<0=auto|1..16>] [group=<g>]   (ping-pong tiles: 256x256 for
//          bf16 / fp16 / int8, 256x128 for block FP8; split only for block FP8)
//   decode swap=<0|1> split=<0=auto|1..256> reduce=<lastwg|atomic|twopass>
//          waves=<w> unroll=<u> rows=<weight rows per workgroup, 4..64, 4 | rows>
// The first matching entry wins.
#pragma once

#include <string>
#include <vector>

#include "launch.hpp"

namespace lg {

struct TableEntry {
  int quant;  // -1 = any
  long long m_lo, m_hi;  // m_hi -1 = no bound
  long long n, k;        // -1 = any
  Variant v;
};

// Parse a variant spec; returns false with a message on error.
bool parse_variant(const std::string& spec, Variant* out, std::string* err);
// Render a variant (with split resolved by the caller if wanted).
std::string format_variant(const Variant& v, int split);
// Parse a whole table text.
bool parse_table(const std::string& text, std::vector<TableEntry>* out, std::string* err);
// The built-in table.
const char* builtin_table();
// First matching entry; false if none matches.
bool lookup(const std::vector<TableEntry>& t, int quant, long long M, long long N, long long K,
            Variant* out);

}  // namespace lg
