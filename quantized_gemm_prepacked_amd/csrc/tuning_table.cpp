// tuning_table.cpp -- a tuning table loaded at run time, ahead of the built-in per-M-range table.
//
// The Humming announcement (section "Tuning and JIT compilation per workload") prepares kernel
// configurations per range of input sizes and picks one at run time by heuristics; its roadmap
// (section "Roadmap", "Adding autotune") adds benchmarking candidate configurations on the
// target device. Here the benchmarking is offline (quantized_gemm_prepacked_amd/autotune.py) and
// its result is a text table, one entry per line:
//     <family> <asym 0|1> <N> <K> <max_m> <kind> <cfg> <split>
// family = wna16 | w8a8 | w4a8 | w4a4 | w4a8mx | mxw4a16 | fp8b; kind 0 skinny, 1 LDS-tiled, 2 async-pipelined,
// 3 ping-pong; split = K splits of the skinny kernel (-1 = the heuristic's). For a dense call the
// first entry of its (family, asym, N, K) whose max_m covers M is used when that configuration
// fits the shape; otherwise the built-in table decides. '#' starts a comment.
#include <cstdio>
#include <cstdlib>
#include <fstream>
#include <mutex>
#include <sstream>
#include <string>
#include <vector>

#include "internal.h"

namespace hq {

namespace {

struct TuneEntry {
  Family fam;
  bool asym;
  int64_t N, K, max_m;
  int kind, cfg, split;
};

std::mutex g_mu;
std::vector<TuneEntry> g_table;
bool g_loaded = false;   // set by an explicit load (or clear), or after the environment's file

bool parse_family(const std::string& s, Family* f) {
  if (s == "wna16") *f = FAM_WNA16;
  else if (s == "w8a8") *f = FAM_W8A8;
  else if (s == "w4a8") *f = FAM_W4A8;
  else if (s == "w4a4") *f = FAM_W4A4;
  else if (s == "w4a8mx") *f = FAM_W4A8MX;
  else if (s == "mxw4a16") *f = FAM_MXW4A16;
  else if (s == "fp8b") *f = FAM_FP8B;
  else if (s == "w8a16") *f = FAM_W8A16;
  else if (s == "f8a16") *f = FAM_F8A16;
  else if (s == "wna2") *f = FAM_WNA2;
  else if (s == "wna3") *f = FAM_WNA3;
  else return false;
  return true;
}

int parse_file(const char* path, std::vector<TuneEntry>* out, std::string* err) {
  std::ifstream in(path);
  if (!in) {
    *err = std::string("cannot open tuning table '") + path + "'";
    return 1;
  }
  std::string line;
  int lineno = 0;
  while (std::getline(in, line)) {
    ++lineno;
    const size_t hash = line.find('#');
    if (hash != std::string::npos) line.resize(hash);
    std::istringstream ss(line);
    std::string fam;
    if (!(ss >> fam)) continue;   // blank or comment
    TuneEntry e{};
    int asym = 0;
    std::string extra;
    if (!parse_family(fam, &e.fam) || !(ss >> asym >> e.N >> e.K >> e.max_m >> e.kind >> e.cfg >> e.split) ||
        (ss >> extra) || asym < 0 || asym > 1 || e.N <= 0 || e.K <= 0 || e.max_m <= 0 || e.kind < 0 ||
        e.kind > 3 || e.cfg < 0 || e.split == 0 || e.split < -1) {
      char buf[160];
      std::snprintf(buf, sizeof(buf), "tuning table '%s' line %d: expected '<family> <asym> <N> <K> <max_m> "
                    "<kind> <cfg> <split>'", path, lineno);
      *err = buf;
      return 1;
    }
    e.asym = asym != 0;
    out->push_back(e);
  }
  return 0;
}

}  // namespace

int load_tuning_table(const char* path, std::string* err) {
  std::vector<TuneEntry> t;
  if (path && parse_file(path, &t, err) != 0) return 1;
  std::lock_guard<std::mutex> lk(g_mu);
  g_table.swap(t);
  g_loaded = true;
  return 0;
}

bool tuning_lookup(const Combo& c, int64_t M, int64_t N, int64_t K, int* kind, int* cfg, int* split) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_loaded) {
    g_loaded = true;
    if (const char* p = std::getenv("HQ_TUNING_FILE")) {
      std::string err;
      std::vector<TuneEntry> t;
      if (parse_file(p, &t, &err) == 0) g_table.swap(t);   // an unreadable file leaves it empty
    }
  }
  for (const TuneEntry& e : g_table) {
    if (e.fam != c.fam || e.asym != c.asym || e.N != N || e.K != K || M > e.max_m) continue;
    *kind = e.kind;
    *cfg = e.cfg;
    *split = e.split;
    return true;
  }
  return false;
}

}  // namespace hq
