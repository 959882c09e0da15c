// ks_oracle.cpp -- CPU oracle for the PTX-subset SIMT simulator.
//
// TEST INFRASTRUCTURE ONLY: a plain, slow, obviously correct interpreter used to
// check the GPU simulator.  Only the tests, the smoke check and the benchmark's
// CPU-baseline leg may load it; the product path must never route through it.
// It shares no code with the GPU path (own parser, own post-dominators, own copy
// of the output layouts).  Build with -ffp-contract=off and without fast-math:
// single-precision results are compared bit for bit.
//
// Sources of the semantics (cited by page title and section):
//  * KernelScope backend documentation (github.com/briefgaming/kernelscope):
//    - "PTX Parser" part (ptx/parser.py): module directives, entry/param/reg
//      declarations and the instruction grammar (optional @/@! guard, opcode,
//      dotted modifiers, comma-separated operands, trailing comment).
//    - "Execution Simulator" part (simulator/models.py): per-thread registers and
//      predicates, the 32-thread warp with a 32-bit active mask and a SIMT stack of
//      (pc, mask, reconvergence pc) entries, if/else divergence executed serially
//      with complementary masks and reconverging to the union, the block with a
//      zero-filled shared window and a barrier.
//    - "Memory analysis" part (simulator/engine.py): 32 banks of 4 bytes,
//      bank = (address / 4) mod 32, a bank whose threads all use one address is a
//      broadcast, conflict degree = largest thread count of a non-broadcast bank;
//      128-byte lines and 32-byte sectors for global accesses.
//    - "Latency model" part (latency/model.py): sm_80 latencies (int/fp32 4,
//      ld.global 200, ld.shared 23, ld.const 4, bra 4, bar.sync 20).
//  * "CuTeDSL IKET 浅析" (zhen8838.github.io/posts/iket.html), section 2,
//    "buffer 是怎么定形的": one trace slot per warp, a 16-byte header, fixed-size
//    records, a per-warp record cap with overflow counted as missed.
//  * The cycle rule (issue at the later of previous issue + 1 and the ready cycle
//    of every source) is the register-scoreboard reading of the dependent versus
//    independent FFMA contrast in the SASS-probe method page
//    (teach-meaning.tistory.com/1954), sections 2 and 14.
// Where the pages are silent the readings taken are listed in the design notes
// of the repository and restated at the point of use below.

#include "ks_oracle.h"

#include <algorithm>
#include <atomic>
#include <cctype>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <set>
#include <stdexcept>
#include <string>
#include <thread>
#include <vector>
#include <xmmintrin.h>

namespace {

// ---------------------------------------------------------------- errors

struct OracleError {
  int code;
  std::string msg;
};

[[noreturn]] void fail(int code, int line, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  std::string m = line > 0 ? ("line " + std::to_string(line) + ": " + buf) : std::string(buf);
  throw OracleError{code, m};
}

void set_err(char* err, size_t err_len, const std::string& m) {
  if (err && err_len) {
    size_t k = std::min(err_len - 1, m.size());
    memcpy(err, m.data(), k);
    err[k] = 0;
  }
}

// ---------------------------------------------------------------- program model

enum RegClass { RC_32, RC_64, RC_PRED };

struct RegDecl {
  std::string name;
  RegClass cls;
  int index;  // index into the per-lane value array (RC_32/RC_64) or predicate array
};

enum OperandKind { K_NONE, K_REG, K_PRED, K_IMM, K_SPECIAL };

enum Special {
  SP_TID_X, SP_TID_Y, SP_TID_Z, SP_NTID_X, SP_NTID_Y, SP_NTID_Z,
  SP_CTAID_X, SP_CTAID_Y, SP_CTAID_Z, SP_NCTAID_X, SP_NCTAID_Y, SP_NCTAID_Z, SP_LANEID
};

struct Operand {
  OperandKind kind = K_NONE;
  int reg = -1;       // value index (K_REG) or predicate index (K_PRED)
  int width = 0;      // 32 or 64 for K_REG
  uint64_t imm = 0;   // K_IMM
  int special = -1;   // K_SPECIAL
};

enum Op {
  OP_ADD, OP_SUB, OP_MUL_LO, OP_MUL_WIDE, OP_MAD_LO,
  OP_FADD, OP_FSUB, OP_FMUL, OP_FFMA,
  OP_SETP, OP_SELP, OP_MOV,
  OP_LD_PARAM, OP_LD_GLOBAL, OP_LD_SHARED, OP_ST_GLOBAL, OP_ST_SHARED,
  OP_BRA, OP_BAR, OP_RET
};

enum Cmp { CMP_EQ, CMP_NE, CMP_LT, CMP_LE, CMP_GT, CMP_GE };

struct Inst {
  int line = 0;
  Op op = OP_RET;
  int width = 32;        // operand width of the instruction type (32 or 64)
  bool is_signed = false;
  bool is_float = false;
  bool bits_only = false;  // .bN type (setp allows eq/ne only)
  Cmp cmp = CMP_EQ;
  bool has_guard = false;
  bool guard_neg = false;
  int guard_pred = -1;
  Operand dst;
  Operand src[3];
  int nsrc = 0;
  // memory operand
  int addr_reg = -1;
  int addr_width = 0;
  int64_t addr_off = 0;
  uint32_t param_off = 0;
  int size = 0;          // access size in bytes
  int target = -1;       // branch target index
  int lat_class = ORACLE_LAT_INT32;
};

struct Param {
  std::string name;
  uint32_t size = 0;
  uint32_t offset = 0;
};

struct Program {
  std::vector<Inst> code;
  std::vector<Param> params;
  uint32_t param_bytes = 0;
  uint32_t shared_bytes = 0;
  int n_vals = 0;   // value slots (one per 32- or 64-bit register)
  int n_preds = 0;
  uint32_t reg_words = 0;
  std::vector<uint32_t> rpc;  // reconvergence index per instruction (EXIT_PC if exit)
};

const uint32_t EXIT_PC = 0xFFFFFFFFu;

// ---------------------------------------------------------------- text helpers

std::string trim(const std::string& s) {
  size_t a = 0, b = s.size();
  while (a < b && isspace((unsigned char)s[a])) ++a;
  while (b > a && isspace((unsigned char)s[b - 1])) --b;
  return s.substr(a, b - a);
}

bool starts_with(const std::string& s, const std::string& p) {
  return s.size() >= p.size() && s.compare(0, p.size(), p) == 0;
}

std::vector<std::string> split_dots(const std::string& s) {
  std::vector<std::string> out;
  std::string cur;
  for (char c : s) {
    if (c == '.') {
      out.push_back(cur);
      cur.clear();
    } else {
      cur += c;
    }
  }
  out.push_back(cur);
  return out;
}

bool is_ident_char(char c) { return isalnum((unsigned char)c) || c == '_' || c == '$'; }

// Statement = one ';'-terminated piece of text, a label, or a brace.
struct Stmt {
  int line;
  std::string text;
};

// Strip comments, drop .loc/.file lines (they carry no ';'), split into statements.
std::vector<Stmt> split_statements(const std::string& src) {
  // 1. remove comments, keeping newlines so line numbers survive
  std::string t;
  t.reserve(src.size());
  for (size_t i = 0; i < src.size();) {
    if (src[i] == '/' && i + 1 < src.size() && src[i + 1] == '/') {
      while (i < src.size() && src[i] != '\n') ++i;
    } else if (src[i] == '/' && i + 1 < src.size() && src[i + 1] == '*') {
      i += 2;
      while (i + 1 < src.size() && !(src[i] == '*' && src[i + 1] == '/')) {
        if (src[i] == '\n') t += '\n';
        ++i;
      }
      i += 2;
    } else {
      t += src[i++];
    }
  }
  // 2. walk lines
  std::vector<Stmt> out;
  std::string cur;
  int cur_line = 0;
  int line = 1;
  size_t pos = 0;
  while (pos <= t.size()) {
    size_t e = t.find('\n', pos);
    if (e == std::string::npos) e = t.size();
    std::string ln = t.substr(pos, e - pos);
    std::string tl = trim(ln);
    if (starts_with(tl, ".loc") || starts_with(tl, ".file") || starts_with(tl, ".section")) {
      tl.clear();  // source-map directives are ignored
    }
    if (trim(cur).empty() && (starts_with(tl, ".version") || starts_with(tl, ".target") ||
                              starts_with(tl, ".address_size"))) {
      // module directives end at the end of their line
      std::string d = tl;
      if (!d.empty() && d.back() == ';') d.pop_back();
      out.push_back({line, trim(d)});
      tl.clear();
    }
    size_t i = 0;
    while (i < tl.size()) {
      char c = tl[i];
      if (c == ';') {
        if (!trim(cur).empty()) out.push_back({cur_line, trim(cur)});
        cur.clear();
        ++i;
      } else if (c == '{' || c == '}') {
        if (!trim(cur).empty()) {
          // text before a brace (for instance the ')' closing the parameter list)
          out.push_back({cur_line, trim(cur)});
          cur.clear();
        }
        out.push_back({line, std::string(1, c)});
        ++i;
      } else {
        if (trim(cur).empty()) {
          cur.clear();
          cur_line = line;
          // a label "name:" at the start of a statement
          size_t j = i;
          while (j < tl.size() && is_ident_char(tl[j])) ++j;
          if (j > i && j < tl.size() && tl[j] == ':') {
            out.push_back({line, tl.substr(i, j - i + 1)});
            i = j + 1;
            continue;
          }
        }
        cur += c;
        ++i;
      }
    }
    if (!cur.empty()) cur += ' ';
    pos = e + 1;
    ++line;
  }
  if (!trim(cur).empty()) out.push_back({cur_line, trim(cur)});
  return out;
}

// ---------------------------------------------------------------- parser

struct TypeInfo {
  int width;  // 32, 64 or 1 (pred)
  bool is_signed, is_float, bits_only;
};

bool type_of(const std::string& t, TypeInfo& ti) {
  if (t == "s32") ti = {32, true, false, false};
  else if (t == "u32") ti = {32, false, false, false};
  else if (t == "b32") ti = {32, false, false, true};
  else if (t == "f32") ti = {32, false, true, false};
  else if (t == "s64") ti = {64, true, false, false};
  else if (t == "u64") ti = {64, false, false, false};
  else if (t == "b64") ti = {64, false, false, true};
  else if (t == "pred") ti = {1, false, false, false};
  else return false;
  return true;
}

struct Parser {
  Program prog;
  std::map<std::string, RegDecl> regs;
  std::map<std::string, uint32_t> shared_vars;  // name -> byte offset in the window
  std::map<std::string, int> labels;
  std::vector<std::pair<int, std::string>> pending_targets;  // (inst index, label)

  void declare_reg(int line, const std::string& tname, const std::string& name) {
    TypeInfo ti;
    if (!type_of(tname, ti)) fail(ORACLE_E_UNSUPPORTED, line, "unsupported register type .%s", tname.c_str());
    if (regs.count(name)) fail(ORACLE_E_PARSE, line, "register %s declared twice", name.c_str());
    RegDecl d;
    d.name = name;
    if (ti.width == 1) {
      d.cls = RC_PRED;
      d.index = prog.n_preds++;
    } else {
      d.cls = ti.width == 64 ? RC_64 : RC_32;
      d.index = prog.n_vals++;
      prog.reg_words += ti.width / 32;
    }
    regs[name] = d;
  }

  void parse_reg_decl(const Stmt& st) {
    // .reg .type %name<N>   |   .reg .type %a, %b
    std::string rest = trim(st.text.substr(4));
    if (rest.empty() || rest[0] != '.') fail(ORACLE_E_PARSE, st.line, "bad .reg declaration");
    size_t sp = rest.find_first_of(" \t");
    if (sp == std::string::npos) fail(ORACLE_E_PARSE, st.line, "bad .reg declaration");
    std::string tname = rest.substr(1, sp - 1);
    std::string names = trim(rest.substr(sp));
    size_t start = 0;
    while (start <= names.size()) {
      size_t comma = names.find(',', start);
      if (comma == std::string::npos) comma = names.size();
      std::string nm = trim(names.substr(start, comma - start));
      start = comma + 1;
      if (nm.empty()) continue;
      size_t lt = nm.find('<');
      if (lt != std::string::npos) {
        size_t gt = nm.find('>', lt);
        if (gt == std::string::npos) fail(ORACLE_E_PARSE, st.line, "bad register range");
        std::string base = nm.substr(0, lt);
        long cnt = strtol(nm.substr(lt + 1, gt - lt - 1).c_str(), nullptr, 10);
        if (cnt <= 0 || cnt > 100000) fail(ORACLE_E_PARSE, st.line, "bad register count");
        for (long k = 0; k < cnt; ++k) declare_reg(st.line, tname, base + std::to_string(k));
      } else {
        declare_reg(st.line, tname, nm);
      }
    }
  }

  void parse_shared_decl(const Stmt& st) {
    // .shared [.align A] .type name[N]
    std::string rest = trim(st.text.substr(7));
    uint32_t align = 0;
    if (starts_with(rest, ".align")) {
      rest = trim(rest.substr(6));
      size_t sp = rest.find_first_of(" \t");
      if (sp == std::string::npos) fail(ORACLE_E_PARSE, st.line, "bad .shared");
      align = (uint32_t)strtoul(rest.substr(0, sp).c_str(), nullptr, 10);
      rest = trim(rest.substr(sp));
    }
    if (rest.empty() || rest[0] != '.') fail(ORACLE_E_PARSE, st.line, "bad .shared");
    size_t sp = rest.find_first_of(" \t");
    if (sp == std::string::npos) fail(ORACLE_E_PARSE, st.line, "bad .shared");
    std::string tname = rest.substr(1, sp - 1);
    uint32_t esize;
    if (tname == "b8" || tname == "u8" || tname == "s8") esize = 1;
    else if (tname == "b16" || tname == "u16" || tname == "s16") esize = 2;
    else if (tname == "b32" || tname == "u32" || tname == "s32" || tname == "f32") esize = 4;
    else if (tname == "b64" || tname == "u64" || tname == "s64") esize = 8;
    else fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported .shared type");
    std::string decl = trim(rest.substr(sp));
    size_t lb = decl.find('[');
    uint64_t count = 1;
    std::string name = decl;
    if (lb != std::string::npos) {
      size_t rb = decl.find(']', lb);
      if (rb == std::string::npos) fail(ORACLE_E_PARSE, st.line, "bad .shared array");
      name = trim(decl.substr(0, lb));
      count = strtoull(decl.substr(lb + 1, rb - lb - 1).c_str(), nullptr, 10);
    }
    if (align == 0) align = esize;
    if (align & (align - 1)) fail(ORACLE_E_PARSE, st.line, "alignment must be a power of two");
    uint64_t off = (prog.shared_bytes + align - 1) / align * align;
    uint64_t end = off + count * esize;
    if (end > (1u << 20)) fail(ORACLE_E_UNSUPPORTED, st.line, "shared window too large");
    shared_vars[name] = (uint32_t)off;
    prog.shared_bytes = (uint32_t)end;
  }

  void parse_params(const std::string& plist, int line) {
    size_t start = 0;
    uint32_t off = 0;
    while (start < plist.size()) {
      size_t comma = plist.find(',', start);
      if (comma == std::string::npos) comma = plist.size();
      std::string p = trim(plist.substr(start, comma - start));
      start = comma + 1;
      if (p.empty()) continue;
      if (!starts_with(p, ".param")) fail(ORACLE_E_PARSE, line, "expected .param");
      std::string rest = trim(p.substr(6));
      if (rest.empty() || rest[0] != '.') fail(ORACLE_E_PARSE, line, "bad .param");
      size_t sp = rest.find_first_of(" \t");
      if (sp == std::string::npos) fail(ORACLE_E_PARSE, line, "bad .param");
      TypeInfo ti;
      if (!type_of(rest.substr(1, sp - 1), ti) || ti.width == 1)
        fail(ORACLE_E_UNSUPPORTED, line, "unsupported .param type");
      Param pr;
      pr.name = trim(rest.substr(sp));
      pr.size = (uint32_t)(ti.width / 8);
      off = (off + pr.size - 1) / pr.size * pr.size;  // natural alignment, declaration order
      pr.offset = off;
      off += pr.size;
      prog.params.push_back(pr);
    }
    prog.param_bytes = off;
  }

  // ---- operands

  bool parse_int_literal(const std::string& s, uint64_t& v) {
    std::string t = s;
    bool neg = false;
    if (!t.empty() && (t[0] == '-' || t[0] == '+')) {
      neg = t[0] == '-';
      t = t.substr(1);
    }
    if (t.empty()) return false;
    uint64_t x = 0;
    if (t.size() > 2 && t[0] == '0' && (t[1] == 'x' || t[1] == 'X')) {
      for (size_t i = 2; i < t.size(); ++i) {
        char c = (char)tolower((unsigned char)t[i]);
        int d;
        if (c >= '0' && c <= '9') d = c - '0';
        else if (c >= 'a' && c <= 'f') d = c - 'a' + 10;
        else return false;
        if (x >> 60) return false;
        x = x * 16 + (uint64_t)d;
      }
    } else {
      for (char c : t) {
        if (c < '0' || c > '9') return false;
        uint64_t nx = x * 10 + (uint64_t)(c - '0');
        if (nx / 10 != x) return false;
        x = nx;
      }
    }
    v = neg ? (uint64_t)(0 - x) : x;
    return true;
  }

  bool parse_f32_literal(const std::string& s, uint64_t& v) {
    if (s.size() != 10 || s[0] != '0' || (s[1] != 'f' && s[1] != 'F')) return false;
    uint64_t x = 0;
    for (size_t i = 2; i < 10; ++i) {
      char c = (char)tolower((unsigned char)s[i]);
      int d;
      if (c >= '0' && c <= '9') d = c - '0';
      else if (c >= 'a' && c <= 'f') d = c - 'a' + 10;
      else return false;
      x = x * 16 + (uint64_t)d;
    }
    v = x;
    return true;
  }

  int special_of(const std::string& s) {
    static const char* names[] = {"%tid.x", "%tid.y", "%tid.z", "%ntid.x", "%ntid.y", "%ntid.z",
                                  "%ctaid.x", "%ctaid.y", "%ctaid.z", "%nctaid.x", "%nctaid.y",
                                  "%nctaid.z", "%laneid"};
    for (int i = 0; i < 13; ++i)
      if (s == names[i]) return i;
    return -1;
  }

  // A value source of the given width: register, immediate or (when allowed) special register.
  Operand value_operand(int line, const std::string& s, int width, bool is_float, bool allow_special) {
    Operand o;
    auto it = regs.find(s);
    if (it != regs.end()) {
      if (it->second.cls == RC_PRED) fail(ORACLE_E_PARSE, line, "predicate %s used as a value", s.c_str());
      int w = it->second.cls == RC_64 ? 64 : 32;
      if (w != width) fail(ORACLE_E_PARSE, line, "register %s has width %d, expected %d", s.c_str(), w, width);
      o.kind = K_REG;
      o.reg = it->second.index;
      o.width = w;
      return o;
    }
    if (!s.empty() && s[0] == '%') {
      int sp = special_of(s);
      if (sp >= 0) {
        if (!allow_special) fail(ORACLE_E_UNSUPPORTED, line, "special register %s only allowed in mov", s.c_str());
        if (width != 32) fail(ORACLE_E_PARSE, line, "special registers are 32-bit");
        o.kind = K_SPECIAL;
        o.special = sp;
        return o;
      }
      fail(ORACLE_E_PARSE, line, "undeclared register %s", s.c_str());
    }
    uint64_t v;
    if (parse_f32_literal(s, v)) {
      if (width != 32) fail(ORACLE_E_PARSE, line, "0f literal in a 64-bit operand");
      o.kind = K_IMM;
      o.imm = v;
      return o;
    }
    if (is_float) {
      if (!s.empty() && (isdigit((unsigned char)s[0]) || s[0] == '-' || s[0] == '+'))
        fail(ORACLE_E_UNSUPPORTED, line, "f32 immediates must be written as 0fXXXXXXXX bit patterns");
    }
    if (!is_float && parse_int_literal(s, v)) {
      o.kind = K_IMM;
      if (width == 32) {
        int64_t sv = (int64_t)v;
        bool neg = !s.empty() && s[0] == '-';
        if (neg ? (sv < -2147483648LL) : (v > 0xFFFFFFFFull))
          fail(ORACLE_E_PARSE, line, "immediate %s does not fit 32 bits", s.c_str());
        o.imm = v & 0xFFFFFFFFull;
      } else {
        o.imm = v;
      }
      return o;
    }
    auto sv = shared_vars.find(s);
    if (sv != shared_vars.end() && allow_special && !is_float) {
      o.kind = K_IMM;  // address of a shared variable = its offset in the window
      o.imm = sv->second;
      return o;
    }
    fail(ORACLE_E_PARSE, line, "bad operand '%s'", s.c_str());
  }

  Operand dst_operand(int line, const std::string& s, int width) {
    auto it = regs.find(s);
    if (it == regs.end()) fail(ORACLE_E_PARSE, line, "undeclared destination %s", s.c_str());
    if (it->second.cls == RC_PRED) fail(ORACLE_E_PARSE, line, "predicate %s used as a value", s.c_str());
    int w = it->second.cls == RC_64 ? 64 : 32;
    if (w != width) fail(ORACLE_E_PARSE, line, "register %s has width %d, expected %d", s.c_str(), w, width);
    Operand o;
    o.kind = K_REG;
    o.reg = it->second.index;
    o.width = w;
    return o;
  }

  Operand pred_operand(int line, const std::string& s) {
    auto it = regs.find(s);
    if (it == regs.end() || it->second.cls != RC_PRED) fail(ORACLE_E_PARSE, line, "expected a predicate, got '%s'", s.c_str());
    Operand o;
    o.kind = K_PRED;
    o.reg = it->second.index;
    return o;
  }

  std::vector<std::string> split_operands(const std::string& s) {
    std::vector<std::string> out;
    std::string cur;
    int depth = 0;
    for (char c : s) {
      if (c == '[') ++depth;
      if (c == ']') --depth;
      if (c == ',' && depth == 0) {
        out.push_back(trim(cur));
        cur.clear();
      } else {
        cur += c;
      }
    }
    if (!trim(cur).empty()) out.push_back(trim(cur));
    return out;
  }

  // "[%r]", "[%r+8]", "[%r-8]" for global/shared; "[name]" or "[name+8]" for param.
  void memory_operand(int line, const std::string& s, Inst& in, bool is_param) {
    if (s.size() < 3 || s.front() != '[' || s.back() != ']') fail(ORACLE_E_PARSE, line, "bad address '%s'", s.c_str());
    std::string body = trim(s.substr(1, s.size() - 2));
    std::string base = body;
    int64_t off = 0;
    size_t k = body.find_first_of("+-", 1);
    if (k != std::string::npos) {
      base = trim(body.substr(0, k));
      std::string rest = trim(body.substr(k + 1));
      uint64_t v;
      if (!parse_int_literal(rest, v)) fail(ORACLE_E_PARSE, line, "bad address offset '%s'", rest.c_str());
      off = body[k] == '-' ? -(int64_t)v : (int64_t)v;
    }
    if (is_param) {
      for (const Param& p : prog.params) {
        if (p.name == base) {
          if (off < 0 || (uint64_t)off + (uint64_t)in.size > p.size)
            fail(ORACLE_E_PARSE, line, "param access outside %s", base.c_str());
          in.param_off = p.offset + (uint32_t)off;
          return;
        }
      }
      fail(ORACLE_E_PARSE, line, "unknown parameter %s", base.c_str());
    }
    auto it = regs.find(base);
    if (it == regs.end() || it->second.cls == RC_PRED) fail(ORACLE_E_PARSE, line, "address base must be a register: '%s'", base.c_str());
    in.addr_reg = it->second.index;
    in.addr_width = it->second.cls == RC_64 ? 64 : 32;
    in.addr_off = off;
  }

  void parse_instruction(const Stmt& st) {
    Inst in;
    in.line = st.line;
    std::string s = st.text;
    if (s[0] == '@') {
      size_t sp = s.find_first_of(" \t");
      if (sp == std::string::npos) fail(ORACLE_E_PARSE, st.line, "guard without instruction");
      std::string g = s.substr(1, sp - 1);
      in.has_guard = true;
      if (!g.empty() && g[0] == '!') {
        in.guard_neg = true;
        g = g.substr(1);
      }
      in.guard_pred = pred_operand(st.line, g).reg;
      s = trim(s.substr(sp));
    }
    size_t sp = s.find_first_of(" \t");
    std::string opword = sp == std::string::npos ? s : s.substr(0, sp);
    std::string rest = sp == std::string::npos ? "" : trim(s.substr(sp));
    std::vector<std::string> parts = split_dots(opword);
    std::vector<std::string> ops = split_operands(rest);
    const std::string& base = parts[0];
    auto need = [&](size_t n) {
      if (ops.size() != n) fail(ORACLE_E_PARSE, st.line, "%s expects %zu operands", opword.c_str(), n);
    };
    auto the_type = [&](const std::string& t) {
      TypeInfo ti;
      if (!type_of(t, ti) || ti.width == 1) fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported type .%s in %s", t.c_str(), opword.c_str());
      in.width = ti.width;
      in.is_signed = ti.is_signed;
      in.is_float = ti.is_float;
      in.bits_only = ti.bits_only;
    };
    if (base == "add" || base == "sub") {
      // add.T / sub.T, with an optional .rn on f32
      std::vector<std::string> m(parts.begin() + 1, parts.end());
      bool rn = false;
      if (m.size() == 2 && m[0] == "rn") { rn = true; m.erase(m.begin()); }
      if (m.size() != 1) fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported form %s", opword.c_str());
      the_type(m[0]);
      if (rn && !in.is_float) fail(ORACLE_E_PARSE, st.line, ".rn on an integer add");
      if (in.bits_only) fail(ORACLE_E_UNSUPPORTED, st.line, "%s needs a signed, unsigned or float type", opword.c_str());
      in.op = in.is_float ? (base == "add" ? OP_FADD : OP_FSUB) : (base == "add" ? OP_ADD : OP_SUB);
      in.lat_class = in.is_float ? ORACLE_LAT_FP32 : (in.width == 64 ? ORACLE_LAT_INT64 : ORACLE_LAT_INT32);
      need(3);
      in.dst = dst_operand(st.line, ops[0], in.width);
      in.src[0] = value_operand(st.line, ops[1], in.width, in.is_float, false);
      in.src[1] = value_operand(st.line, ops[2], in.width, in.is_float, false);
      in.nsrc = 2;
    } else if (base == "mul") {
      if (parts.size() == 3 && parts[1] == "lo") {
        the_type(parts[2]);
        if (in.is_float || in.bits_only) fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported form %s", opword.c_str());
        in.op = OP_MUL_LO;
        in.lat_class = in.width == 64 ? ORACLE_LAT_INT64 : ORACLE_LAT_INT32;
        need(3);
        in.dst = dst_operand(st.line, ops[0], in.width);
        in.src[0] = value_operand(st.line, ops[1], in.width, false, false);
        in.src[1] = value_operand(st.line, ops[2], in.width, false, false);
        in.nsrc = 2;
      } else if (parts.size() == 3 && parts[1] == "wide") {
        the_type(parts[2]);
        if (in.is_float || in.bits_only || in.width != 32) fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported form %s", opword.c_str());
        in.op = OP_MUL_WIDE;
        in.lat_class = ORACLE_LAT_INT32;
        need(3);
        in.dst = dst_operand(st.line, ops[0], 64);
        in.src[0] = value_operand(st.line, ops[1], 32, false, false);
        in.src[1] = value_operand(st.line, ops[2], 32, false, false);
        in.nsrc = 2;
      } else if ((parts.size() == 2 && parts[1] == "f32") ||
                 (parts.size() == 3 && parts[1] == "rn" && parts[2] == "f32")) {
        the_type("f32");
        in.op = OP_FMUL;
        in.lat_class = ORACLE_LAT_FP32;
        need(3);
        in.dst = dst_operand(st.line, ops[0], 32);
        in.src[0] = value_operand(st.line, ops[1], 32, true, false);
        in.src[1] = value_operand(st.line, ops[2], 32, true, false);
        in.nsrc = 2;
      } else {
        fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported form %s", opword.c_str());
      }
    } else if (base == "mad") {
      if (!(parts.size() == 3 && parts[1] == "lo")) fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported form %s", opword.c_str());
      the_type(parts[2]);
      if (in.is_float || in.bits_only) fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported form %s", opword.c_str());
      in.op = OP_MAD_LO;
      in.lat_class = in.width == 64 ? ORACLE_LAT_INT64 : ORACLE_LAT_INT32;
      need(4);
      in.dst = dst_operand(st.line, ops[0], in.width);
      for (int k = 0; k < 3; ++k) in.src[k] = value_operand(st.line, ops[k + 1], in.width, false, false);
      in.nsrc = 3;
    } else if (base == "fma") {
      if (!(parts.size() == 3 && parts[1] == "rn" && parts[2] == "f32")) fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported form %s", opword.c_str());
      the_type("f32");
      in.op = OP_FFMA;
      in.lat_class = ORACLE_LAT_FP32;
      need(4);
      in.dst = dst_operand(st.line, ops[0], 32);
      for (int k = 0; k < 3; ++k) in.src[k] = value_operand(st.line, ops[k + 1], 32, true, false);
      in.nsrc = 3;
    } else if (base == "setp") {
      if (parts.size() != 3) fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported form %s", opword.c_str());
      the_type(parts[2]);
      const std::string& c = parts[1];
      bool uns_ok = !in.is_signed && !in.is_float && !in.bits_only;
      if (c == "eq") in.cmp = CMP_EQ;
      else if (c == "ne") in.cmp = CMP_NE;
      else if (c == "lt" && !in.bits_only) in.cmp = CMP_LT;
      else if (c == "le" && !in.bits_only) in.cmp = CMP_LE;
      else if (c == "gt" && !in.bits_only) in.cmp = CMP_GT;
      else if (c == "ge" && !in.bits_only) in.cmp = CMP_GE;
      else if (c == "lo" && uns_ok) in.cmp = CMP_LT;
      else if (c == "ls" && uns_ok) in.cmp = CMP_LE;
      else if (c == "hi" && uns_ok) in.cmp = CMP_GT;
      else if (c == "hs" && uns_ok) in.cmp = CMP_GE;
      else fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported comparison %s", opword.c_str());
      in.op = OP_SETP;
      in.lat_class = ORACLE_LAT_SETP;
      need(3);
      in.dst = pred_operand(st.line, ops[0]);
      in.src[0] = value_operand(st.line, ops[1], in.width, in.is_float, false);
      in.src[1] = value_operand(st.line, ops[2], in.width, in.is_float, false);
      in.nsrc = 2;
    } else if (base == "selp") {
      if (parts.size() != 2) fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported form %s", opword.c_str());
      the_type(parts[1]);
      in.op = OP_SELP;
      in.lat_class = ORACLE_LAT_SELP;
      need(4);
      in.dst = dst_operand(st.line, ops[0], in.width);
      in.src[0] = value_operand(st.line, ops[1], in.width, in.is_float, false);
      in.src[1] = value_operand(st.line, ops[2], in.width, in.is_float, false);
      in.src[2] = pred_operand(st.line, ops[3]);
      in.nsrc = 3;
    } else if (base == "mov") {
      if (parts.size() != 2) fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported form %s", opword.c_str());
      the_type(parts[1]);
      in.op = OP_MOV;
      in.lat_class = ORACLE_LAT_MOV;
      need(2);
      in.dst = dst_operand(st.line, ops[0], in.width);
      in.src[0] = value_operand(st.line, ops[1], in.width, in.is_float, true);
      in.nsrc = 1;
    } else if (base == "ld" || base == "st") {
      if (parts.size() != 3) fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported form %s", opword.c_str());
      const std::string& space = parts[1];
      the_type(parts[2]);
      in.size = in.width / 8;
      need(2);
      if (base == "ld") {
        if (space == "param") { in.op = OP_LD_PARAM; in.lat_class = ORACLE_LAT_LD_PARAM; }
        else if (space == "global") { in.op = OP_LD_GLOBAL; in.lat_class = ORACLE_LAT_LD_GLOBAL; }
        else if (space == "shared") { in.op = OP_LD_SHARED; in.lat_class = ORACLE_LAT_LD_SHARED; }
        else fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported state space .%s", space.c_str());
        in.dst = dst_operand(st.line, ops[0], in.width);
        memory_operand(st.line, ops[1], in, in.op == OP_LD_PARAM);
      } else {
        if (space == "global") { in.op = OP_ST_GLOBAL; in.lat_class = ORACLE_LAT_ST_GLOBAL; }
        else if (space == "shared") { in.op = OP_ST_SHARED; in.lat_class = ORACLE_LAT_ST_SHARED; }
        else fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported state space .%s", space.c_str());
        memory_operand(st.line, ops[0], in, false);
        auto it = regs.find(ops[1]);
        if (it == regs.end() || it->second.cls == RC_PRED) fail(ORACLE_E_UNSUPPORTED, st.line, "store value must be a register");
        in.src[0] = value_operand(st.line, ops[1], in.width, in.is_float, false);
        in.nsrc = 1;
      }
    } else if (base == "bra") {
      if (!(parts.size() == 1 || (parts.size() == 2 && parts[1] == "uni"))) fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported form %s", opword.c_str());
      need(1);
      in.op = OP_BRA;
      in.lat_class = ORACLE_LAT_BRA;
      pending_targets.push_back({(int)prog.code.size(), ops[0]});
    } else if (base == "bar") {
      if (!(parts.size() == 2 && parts[1] == "sync")) fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported form %s", opword.c_str());
      need(1);
      uint64_t v;
      if (!parse_int_literal(ops[0], v) || v != 0) fail(ORACLE_E_UNSUPPORTED, st.line, "only bar.sync 0 is supported");
      if (in.has_guard) fail(ORACLE_E_UNSUPPORTED, st.line, "guarded bar.sync is not supported");
      in.op = OP_BAR;
      in.lat_class = ORACLE_LAT_BAR;
    } else if (base == "ret" || base == "exit") {
      if (parts.size() != 1) fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported form %s", opword.c_str());
      need(0);
      in.op = OP_RET;
      in.lat_class = ORACLE_LAT_RET;
    } else {
      fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported instruction '%s'", opword.c_str());
    }
    prog.code.push_back(in);
  }

  void parse(const std::string& src, const char* entry) {
    std::vector<Stmt> sts = split_statements(src);
    bool found = false;
    size_t i = 0;
    while (i < sts.size()) {
      const Stmt& st = sts[i];
      if (starts_with(st.text, ".version") || starts_with(st.text, ".target") || starts_with(st.text, ".address_size")) {
        ++i;
        continue;
      }
      size_t ep = st.text.find(".entry");
      if (ep == std::string::npos) {
        if (st.text == "{" || st.text == "}") fail(ORACLE_E_PARSE, st.line, "unexpected brace");
        fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported module-level statement '%s'", st.text.c_str());
      }
      // header: [.visible] .entry name ( params ) then '{'
      std::string head = st.text;
      std::string pre = trim(head.substr(0, ep));
      if (!(pre.empty() || pre == ".visible")) fail(ORACLE_E_UNSUPPORTED, st.line, "unsupported linkage '%s'", pre.c_str());
      std::string after = trim(head.substr(ep + 6));
      size_t lp = after.find('(');
      std::string name = trim(lp == std::string::npos ? after : after.substr(0, lp));
      std::string plist;
      if (lp != std::string::npos) {
        size_t rp = after.find(')', lp);
        if (rp == std::string::npos) fail(ORACLE_E_PARSE, st.line, "unterminated parameter list");
        plist = after.substr(lp + 1, rp - lp - 1);
      }
      ++i;
      if (i >= sts.size() || sts[i].text != "{") fail(ORACLE_E_PARSE, st.line, "expected '{' after entry header");
      ++i;
      size_t body_start = i;
      int depth = 1;
      while (i < sts.size() && depth > 0) {
        if (sts[i].text == "{") ++depth;
        if (sts[i].text == "}") --depth;
        ++i;
      }
      if (depth != 0) fail(ORACLE_E_PARSE, st.line, "unterminated entry body");
      size_t body_end = i - 1;
      bool want = !found && (entry == nullptr || entry[0] == 0 || name == entry);
      if (!want) continue;
      found = true;
      parse_params(plist, st.line);
      for (size_t k = body_start; k < body_end; ++k) {
        const Stmt& b = sts[k];
        if (b.text == "{" || b.text == "}") fail(ORACLE_E_UNSUPPORTED, b.line, "nested blocks are not supported");
        if (b.text.back() == ':') {
          std::string lab = b.text.substr(0, b.text.size() - 1);
          if (labels.count(lab)) fail(ORACLE_E_PARSE, b.line, "label %s defined twice", lab.c_str());
          labels[lab] = (int)prog.code.size();
        } else if (starts_with(b.text, ".reg")) {
          parse_reg_decl(b);
        } else if (starts_with(b.text, ".shared")) {
          parse_shared_decl(b);
        } else if (b.text[0] == '.') {
          fail(ORACLE_E_UNSUPPORTED, b.line, "unsupported directive '%s'", b.text.c_str());
        } else {
          parse_instruction(b);
        }
      }
    }
    if (!found) fail(ORACLE_E_PARSE, 0, entry && entry[0] ? "entry not found" : "no .entry in module");
    for (auto& pt : pending_targets) {
      auto it = labels.find(pt.second);
      if (it == labels.end()) fail(ORACLE_E_PARSE, prog.code[pt.first].line, "unknown label %s", pt.second.c_str());
      prog.code[pt.first].target = it->second;
    }
    if (prog.code.size() > 60000) fail(ORACLE_E_UNSUPPORTED, 0, "program too long");
  }
};

// ---------------------------------------------------------------- post-dominators
//
// Instruction-level control-flow graph; node n stands for "exit".  Post-dominator
// sets by the textbook fixed point PD(v) = {v} ∪ ⋂ PD(s) over successors s, starting
// from "all nodes".  The immediate post-dominator of v is the strict post-dominator
// d whose own set equals PD(v) without v.  Nodes that cannot reach exit (endless
// loops) get exit as their reconvergence point.

std::vector<std::vector<int>> successors(const Program& p) {
  int n = (int)p.code.size();
  std::vector<std::vector<int>> succ(n);
  for (int v = 0; v < n; ++v) {
    const Inst& in = p.code[v];
    int next = v + 1;  // v + 1 == n is the exit node
    if (in.op == OP_BRA) {
      succ[v].push_back(in.target);  // target n (label at the end) is exit as well
      if (in.has_guard && in.target != next) succ[v].push_back(next);
    } else if (in.op == OP_RET) {
      succ[v].push_back(n);
      if (in.has_guard && next != n) succ[v].push_back(next);
    } else {
      succ[v].push_back(next);
    }
  }
  return succ;
}

std::vector<uint32_t> compute_rpc(const Program& p) {
  int n = (int)p.code.size();
  int N = n + 1;
  std::vector<std::vector<int>> succ = successors(p);
  // reachability of exit
  std::vector<char> reach(N, 0);
  reach[n] = 1;
  bool changed = true;
  while (changed) {
    changed = false;
    for (int v = 0; v < n; ++v) {
      if (reach[v]) continue;
      for (int s : succ[v])
        if (reach[s]) { reach[v] = 1; changed = true; break; }
    }
  }
  std::vector<std::vector<char>> pd(N, std::vector<char>(N, 1));
  pd[n] = std::vector<char>(N, 0);
  pd[n][n] = 1;
  changed = true;
  while (changed) {
    changed = false;
    for (int v = n - 1; v >= 0; --v) {
      if (!reach[v]) continue;
      std::vector<char> acc(N, 1);
      for (int s : succ[v]) {
        if (!reach[s]) continue;
        for (int k = 0; k < N; ++k) acc[k] = acc[k] && pd[s][k];
      }
      acc[v] = 1;
      if (acc != pd[v]) {
        pd[v] = acc;
        changed = true;
      }
    }
  }
  std::vector<uint32_t> rpc(n, EXIT_PC);
  for (int v = 0; v < n; ++v) {
    if (!reach[v]) continue;
    std::vector<char> strict = pd[v];
    strict[v] = 0;
    for (int d = 0; d < N; ++d) {
      if (!strict[d]) continue;
      if (pd[d] == strict) {
        rpc[v] = d == n ? EXIT_PC : (uint32_t)d;
        break;
      }
    }
  }
  return rpc;
}

Program load(const char* ptx, size_t len, const char* entry) {
  Parser ps;
  ps.parse(std::string(ptx, len), entry);
  ps.prog.rpc = compute_rpc(ps.prog);
  return ps.prog;
}

// ---------------------------------------------------------------- arithmetic

uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
// Any NaN produced by arithmetic is written as the canonical pattern 0x7FFFFFFF.
uint32_t canon(float r) { return std::isnan(r) ? 0x7FFFFFFFu : f2u(r); }

bool compare(const Inst& in, uint64_t a, uint64_t b) {
  if (in.is_float) {
    float x = u2f((uint32_t)a), y = u2f((uint32_t)b);
    bool unordered = std::isnan(x) || std::isnan(y);
    switch (in.cmp) {  // ordered comparisons: false whenever either input is NaN
      case CMP_EQ: return !unordered && x == y;
      case CMP_NE: return !unordered && x != y;
      case CMP_LT: return !unordered && x < y;
      case CMP_LE: return !unordered && x <= y;
      case CMP_GT: return !unordered && x > y;
      case CMP_GE: return !unordered && x >= y;
    }
  }
  if (in.is_signed) {
    int64_t x = in.width == 32 ? (int64_t)(int32_t)(uint32_t)a : (int64_t)a;
    int64_t y = in.width == 32 ? (int64_t)(int32_t)(uint32_t)b : (int64_t)b;
    switch (in.cmp) {
      case CMP_EQ: return x == y;
      case CMP_NE: return x != y;
      case CMP_LT: return x < y;
      case CMP_LE: return x <= y;
      case CMP_GT: return x > y;
      case CMP_GE: return x >= y;
    }
  }
  uint64_t x = in.width == 32 ? (uint32_t)a : a, y = in.width == 32 ? (uint32_t)b : b;
  switch (in.cmp) {
    case CMP_EQ: return x == y;
    case CMP_NE: return x != y;
    case CMP_LT: return x < y;
    case CMP_LE: return x <= y;
    case CMP_GT: return x > y;
    case CMP_GE: return x >= y;
  }
  return false;
}

// ---------------------------------------------------------------- race check (debug)
//
// A race is two accesses to one byte by different threads in one epoch, at least
// one a write, whose outcome depends on their order: two writes of different
// values, or a read and a write that changes the byte.  A write changes the byte
// when it stores a value other than the one the byte held at the epoch's first
// access: a read by another thread could then see either value, whichever order
// the simulation happened to take.  Epoch = the whole run for global memory, one
// barrier interval of one block for shared memory.

struct ByteLog {
  bool seen = false;
  uint8_t init = 0;                                 // value at the epoch's first access
  std::map<uint8_t, std::vector<uint64_t>> writes;  // value -> up to two distinct writers
  std::vector<uint64_t> readers;                    // up to two distinct readers
};

struct RaceLog {
  std::map<uint64_t, ByteLog> bytes;
  bool raced = false;
  std::string first;

  static void add_tid(std::vector<uint64_t>& v, uint64_t t) {
    if (v.size() < 2 && std::find(v.begin(), v.end(), t) == v.end()) v.push_back(t);
  }
  static bool other_than(const std::vector<uint64_t>& v, uint64_t t) {
    for (uint64_t x : v)
      if (x != t) return true;
    return false;
  }
  // `cur` is the byte's value before the access, `val` the value read or written.
  void note(const char* space, uint64_t addr, uint64_t tid, bool is_write, uint8_t val, uint8_t cur) {
    ByteLog& b = bytes[addr];
    if (!b.seen) {
      b.seen = true;
      b.init = cur;
    }
    bool race = false;
    if (is_write) {
      for (auto& kv : b.writes)
        if (kv.first != val && other_than(kv.second, tid)) race = true;
      if (val != b.init && other_than(b.readers, tid)) race = true;
      add_tid(b.writes[val], tid);
    } else {
      for (auto& kv : b.writes)
        if (kv.first != b.init && other_than(kv.second, tid)) race = true;
      add_tid(b.readers, tid);
    }
    if (race && !raced) {
      raced = true;
      char buf[160];
      snprintf(buf, sizeof buf, "race on %s byte 0x%llx (thread %llu)", space,
               (unsigned long long)addr, (unsigned long long)tid);
      first = buf;
    }
  }
};

// ---------------------------------------------------------------- simulation

struct StackEntry {
  uint32_t pc, mask, rpc;
};

struct Warp {
  int index = 0;           // warp index within the block
  uint32_t init_mask = 0;
  uint32_t exited = 0;
  std::vector<StackEntry> stack;
  int64_t prev_issue = -1;
  uint64_t bar_ready = 0;
  bool waiting = false;
  bool done = false;
  uint64_t arrival = 0;
  std::vector<uint64_t> vals;    // [reg][lane]
  std::vector<uint8_t> preds;    // [pred][lane]
  std::vector<uint64_t> ready;   // per value register, then per predicate
  oracle_counters c;
  struct Record {
    uint32_t cycle, pc, kind, active, payload;
  };
  std::vector<Record> records;
  uint64_t dropped = 0;
  // cache-latency model: tag of each set (-1 = empty) and the outcome counts
  std::vector<int64_t> l1, l2;
  uint32_t cache_count[3] = {0, 0, 0};  // L1 hits, L2 hits, misses
};

struct Sim {
  const Program* p;
  const oracle_cfg* cfg;
  const uint8_t* params;
  uint8_t* gmem;
  uint64_t gmem_bytes;
  uint32_t warps_per_block;
  uint32_t threads_per_block;
  RaceLog* global_races = nullptr;  // non-null when checking races (single thread)

  uint16_t lat(int cls) const { return cfg->latency[cls]; }

  uint64_t read_val(const Warp& w, const Operand& o, int lane, const uint32_t special[13]) const {
    switch (o.kind) {
      case K_REG: return w.vals[(size_t)o.reg * 32 + lane];
      case K_IMM: return o.imm;
      case K_SPECIAL: return special[o.special];
      case K_PRED: return w.preds[(size_t)o.reg * 32 + lane];
      default: return 0;
    }
  }

  // Issue cycle of the next instruction: the later of previous issue + 1, the
  // barrier release, and the ready cycle of each register source (guard included).
  uint64_t issue_cycle(const Warp& w, const Inst& in) const {
    uint64_t t = (uint64_t)(w.prev_issue + 1);
    t = std::max(t, w.bar_ready);
    auto src_ready = [&](const Operand& o) {
      if (o.kind == K_REG) t = std::max(t, w.ready[o.reg]);
      if (o.kind == K_PRED) t = std::max(t, w.ready[p->n_vals + o.reg]);
    };
    for (int k = 0; k < in.nsrc; ++k) src_ready(in.src[k]);
    if (in.addr_reg >= 0) t = std::max(t, w.ready[in.addr_reg]);
    if (in.has_guard) t = std::max(t, w.ready[p->n_vals + in.guard_pred]);
    return t;
  }

  bool valid(uint64_t a, uint64_t size, int s) const {
    return a % (uint64_t)s == 0 && a <= size && size - a >= (uint64_t)s;
  }

  // One access of the SimpleCache of the cache model: a hit when the line's set
  // holds that line; a miss installs it.
  static bool cache_access(std::vector<int64_t>& tags, uint64_t line) {
    const size_t set = (size_t)(line % tags.size());
    if (tags[set] == (int64_t)line) return true;
    tags[set] = (int64_t)line;
    return false;
  }

  void run_block(uint64_t block_linear, oracle_counters* out_c, uint8_t* out_trace, uint8_t* out_cache) {
    const Program& P = *p;
    uint32_t gx = cfg->grid[0], gy = cfg->grid[1];
    uint32_t ctaid[3] = {(uint32_t)(block_linear % gx), (uint32_t)((block_linear / gx) % gy),
                         (uint32_t)(block_linear / ((uint64_t)gx * gy))};
    std::vector<uint8_t> shared(P.shared_bytes, 0);
    std::unique_ptr<RaceLog> shared_races;
    if (global_races) shared_races.reset(new RaceLog());

    std::vector<Warp> warps(warps_per_block);
    for (uint32_t wi = 0; wi < warps_per_block; ++wi) {
      Warp& w = warps[wi];
      w.index = (int)wi;
      for (int l = 0; l < 32; ++l)
        if (wi * 32 + (uint32_t)l < threads_per_block) w.init_mask |= 1u << l;
      w.stack.push_back({0, w.init_mask, EXIT_PC});
      w.vals.assign((size_t)P.n_vals * 32, 0);
      w.preds.assign((size_t)P.n_preds * 32, 0);
      w.ready.assign((size_t)P.n_vals + P.n_preds, 0);
      memset(&w.c, 0, sizeof w.c);
      w.c.max_stack_depth = 1;
      if (cfg->flags & ORACLE_FLAG_CACHE) {
        w.l1.assign(ORACLE_CACHE_L1_LINES, -1);
        w.l2.assign(ORACLE_CACHE_L2_LINES, -1);
      }
    }

    while (true) {
      for (Warp& w : warps)
        if (!w.done && !w.waiting) run_warp(w, block_linear, ctaid, shared, shared_races.get());
      bool all_done = true;
      uint64_t release = 0;
      for (Warp& w : warps) {
        if (!w.done) {
          all_done = false;
          release = std::max(release, w.arrival);
        }
      }
      if (all_done) break;
      // Every unfinished warp is now waiting: release them together.
      release += lat(ORACLE_LAT_BAR);
      for (Warp& w : warps) {
        if (!w.done) {
          w.waiting = false;
          w.bar_ready = release;
        }
      }
      if (shared_races) {
        if (shared_races->raced && !global_races->raced) {
          global_races->raced = true;
          global_races->first = shared_races->first;
        }
        shared_races.reset(new RaceLog());
      }
    }
    if (shared_races && shared_races->raced && !global_races->raced) {
      global_races->raced = true;
      global_races->first = shared_races->first;
    }

    const bool ext = (cfg->flags & ORACLE_FLAG_EXT_TRACE) != 0;
    const size_t rec = ext ? 16 : 8;
    size_t slot = 16 + rec * (size_t)cfg->trace_cap;
    for (uint32_t wi = 0; wi < warps_per_block; ++wi) {
      Warp& w = warps[wi];
      w.c.cycles = (uint32_t)(w.prev_issue + 1);
      w.c.stall_cycles = w.c.cycles - w.c.warp_instrs;
      if (w.dropped) w.c.status |= ORACLE_ST_TRACE_DROP;
      out_c[wi] = w.c;
      uint8_t* s = out_trace + slot * wi;
      uint32_t written = (uint32_t)w.records.size();
      uint8_t version = ext ? 2 : 1;
      uint8_t flags = (uint8_t)((w.dropped ? 1 : 0) | ((w.c.status & ORACLE_ST_FAULT) ? 2 : 0) |
                                ((w.c.status & ORACLE_ST_BUDGET) ? 4 : 0) |
                                ((w.c.status & ORACLE_ST_FINISHED) ? 8 : 0));
      uint16_t wib = (uint16_t)wi;
      uint64_t dropped = w.dropped;
      memcpy(s + 0, &written, 4);
      memcpy(s + 4, &version, 1);
      memcpy(s + 5, &flags, 1);
      memcpy(s + 6, &wib, 2);
      memcpy(s + 8, &dropped, 8);
      for (uint32_t k = 0; k < written; ++k) {
        const Warp::Record& r = w.records[k];
        uint8_t* d = s + 16 + rec * (size_t)k;
        memcpy(d, &r.cycle, 4);
        if (!ext) {
          memcpy(d + 4, &r.pc, 4);
          continue;
        }
        uint16_t pc16 = (uint16_t)r.pc;
        uint8_t kind = (uint8_t)r.kind, zero = 0;
        memcpy(d + 4, &pc16, 2);
        memcpy(d + 6, &kind, 1);
        memcpy(d + 7, &zero, 1);
        memcpy(d + 8, &r.active, 4);
        memcpy(d + 12, &r.payload, 4);
      }
      // records past records_written are left as they were in the caller's buffer
      if (cfg->flags & ORACLE_FLAG_CACHE) {
        uint8_t* cw = out_cache + (size_t)ORACLE_CACHE_WARP_BYTES * wi;
        const uint32_t head[4] = {w.cache_count[0], w.cache_count[1], w.cache_count[2], 0};
        memcpy(cw, head, 16);
        uint32_t* tags = (uint32_t*)(cw + 16);
        for (uint32_t k = 0; k < ORACLE_CACHE_L1_LINES; ++k) tags[k] = (uint32_t)(w.l1[k] + 1);
        for (uint32_t k = 0; k < ORACLE_CACHE_L2_LINES; ++k) tags[ORACLE_CACHE_L1_LINES + k] = (uint32_t)(w.l2[k] + 1);
      }
    }
  }

  void run_warp(Warp& w, uint64_t block_linear, const uint32_t ctaid[3], std::vector<uint8_t>& shared,
                RaceLog* shared_races) {
    const Program& P = *p;
    const uint32_t n = (uint32_t)P.code.size();
    while (true) {
      // Find the runnable top of the divergence stack.
      uint32_t m = 0;
      while (!w.stack.empty()) {
        StackEntry& top = w.stack.back();
        m = top.mask & ~w.exited;
        if (m == 0 || top.pc == top.rpc) {
          w.stack.pop_back();
          continue;
        }
        if (top.pc >= n) {  // ran off the end of the program: those lanes exit, at no cost
          w.exited |= m;
          continue;
        }
        break;
      }
      if (w.stack.empty()) {
        w.c.status |= ORACLE_ST_FINISHED;
        w.done = true;
        return;
      }
      if (w.c.warp_instrs >= cfg->max_warp_instrs) {
        w.c.status |= ORACLE_ST_BUDGET;
        w.done = true;
        return;
      }
      StackEntry& top = w.stack.back();
      const uint32_t pc = top.pc;
      const Inst& in = P.code[pc];
      uint64_t issue = issue_cycle(w, in);
      if (issue > 0x7FFFFFFFull) {
        w.c.status |= ORACLE_ST_CYCLE_OVF;
        w.done = true;
        return;
      }
      // Issue: trace record (kind and payload filled in below), counters.
      Warp::Record* rec = nullptr;
      if (w.records.size() < cfg->trace_cap) {
        w.records.push_back({(uint32_t)issue, pc, (uint32_t)ORACLE_EV_OTHER, m, 0});
        rec = &w.records.back();
      } else {
        w.dropped++;
      }
      w.c.warp_instrs++;
      w.c.thread_instrs += (uint64_t)__builtin_popcount(m);
      w.prev_issue = (int64_t)issue;

      // Lanes whose guard holds.
      uint32_t g = m;
      if (in.has_guard) {
        g = 0;
        for (int l = 0; l < 32; ++l) {
          if (!((m >> l) & 1)) continue;
          bool pv = w.preds[(size_t)in.guard_pred * 32 + l] != 0;
          if (pv != in.guard_neg) g |= 1u << l;
        }
      }

      uint32_t special[13];
      special[SP_NTID_X] = cfg->block[0];
      special[SP_NTID_Y] = cfg->block[1];
      special[SP_NTID_Z] = cfg->block[2];
      special[SP_CTAID_X] = ctaid[0];
      special[SP_CTAID_Y] = ctaid[1];
      special[SP_CTAID_Z] = ctaid[2];
      special[SP_NCTAID_X] = cfg->grid[0];
      special[SP_NCTAID_Y] = cfg->grid[1];
      special[SP_NCTAID_Z] = cfg->grid[2];

      uint32_t next_pc = pc + 1;
      uint32_t kind = ORACLE_EV_OTHER, payload = g;
      uint32_t dst_lat = lat(in.lat_class);  // the cache model may change a global load's
      switch (in.op) {
        case OP_ADD: case OP_SUB: case OP_MUL_LO: case OP_MUL_WIDE: case OP_MAD_LO:
        case OP_FADD: case OP_FSUB: case OP_FMUL: case OP_FFMA:
        case OP_SETP: case OP_SELP: case OP_MOV:
          for (int l = 0; l < 32; ++l) {
            if (!((g >> l) & 1)) continue;
            uint32_t t = (uint32_t)w.index * 32 + (uint32_t)l;
            special[SP_TID_X] = t % cfg->block[0];
            special[SP_TID_Y] = (t / cfg->block[0]) % cfg->block[1];
            special[SP_TID_Z] = t / (cfg->block[0] * cfg->block[1]);
            special[SP_LANEID] = (uint32_t)l;
            execute_alu(w, in, l, special);
          }
          break;
        case OP_LD_PARAM: {
          uint64_t v = 0;
          memcpy(&v, params + in.param_off, (size_t)in.size);
          for (int l = 0; l < 32; ++l)
            if ((g >> l) & 1) w.vals[(size_t)in.dst.reg * 32 + l] = v;
          break;
        }
        case OP_LD_GLOBAL: case OP_ST_GLOBAL: case OP_LD_SHARED: case OP_ST_SHARED: {
          const MemInfo mi = memory_access(w, in, g, block_linear, shared, shared_races);
          if (in.op == OP_LD_GLOBAL && mi.cached) dst_lat = mi.cache_latency;
          const bool global = in.op == OP_LD_GLOBAL || in.op == OP_ST_GLOBAL;
          const bool load = in.op == OP_LD_GLOBAL || in.op == OP_LD_SHARED;
          kind = global ? (load ? ORACLE_EV_LD_GLOBAL : ORACLE_EV_ST_GLOBAL)
                        : (load ? ORACLE_EV_LD_SHARED : ORACLE_EV_ST_SHARED);
          const uint32_t lanes_g = (uint32_t)__builtin_popcount(g);
          payload = global ? (mi.sectors | (mi.lines << 8) | (lanes_g << 16) | (mi.faults << 24))
                           : (mi.degree | (lanes_g << 16) | (mi.faults << 24));
          break;
        }
        case OP_BRA: {
          uint32_t taken = g, not_taken = m & ~g;
          kind = ORACLE_EV_BRANCH;
          if (not_taken == 0) {
            next_pc = (uint32_t)in.target;
          } else if (taken == 0) {
            next_pc = pc + 1;
          } else {
            // Divergence: the current entry becomes the reconvergence entry; the
            // taken path is pushed first so that the fall-through path runs first.
            uint32_t r = P.rpc[pc];
            uint32_t tgt = (uint32_t)in.target;
            top.pc = r;
            w.c.diverge_n++;
            kind = ORACLE_EV_DIVERGE;
            if (tgt != r) w.stack.push_back({tgt, taken, r});
            if (pc + 1 != r) w.stack.push_back({pc + 1, not_taken, r});
            w.c.max_stack_depth = std::max<uint32_t>(w.c.max_stack_depth, (uint32_t)w.stack.size());
            if (w.stack.size() > 63) fail(ORACLE_E_INVALID_ARG, in.line, "divergence stack deeper than 63");
            next_pc = EXIT_PC;  // pc already updated
          }
          break;
        }
        case OP_RET:
          w.exited |= g;
          kind = ORACLE_EV_RET;
          break;
        case OP_BAR:
          kind = ORACLE_EV_BARRIER;
          payload = 0;
          w.c.barrier_n++;
          if (m != (w.init_mask & ~w.exited)) w.c.status |= ORACLE_ST_BARDIV;
          w.waiting = true;
          w.arrival = issue;
          break;
      }
      if (rec) {
        rec->kind = kind;
        rec->payload = payload;
      }
      if (next_pc != EXIT_PC) w.stack.back().pc = next_pc;

      // Destination ready time, whether or not any lane passed the guard.
      switch (in.op) {
        case OP_ADD: case OP_SUB: case OP_MUL_LO: case OP_MUL_WIDE: case OP_MAD_LO:
        case OP_FADD: case OP_FSUB: case OP_FMUL: case OP_FFMA:
        case OP_SELP: case OP_MOV: case OP_LD_PARAM: case OP_LD_GLOBAL: case OP_LD_SHARED:
          w.ready[in.dst.reg] = issue + dst_lat;
          break;
        case OP_SETP:
          w.ready[P.n_vals + in.dst.reg] = issue + lat(in.lat_class);
          break;
        default:
          break;
      }
      if (w.waiting) return;
    }
  }

  void execute_alu(Warp& w, const Inst& in, int l, const uint32_t special[13]) {
    uint64_t a = read_val(w, in.src[0], l, special);
    uint64_t b = in.nsrc > 1 ? read_val(w, in.src[1], l, special) : 0;
    uint64_t c = in.nsrc > 2 ? read_val(w, in.src[2], l, special) : 0;
    uint64_t mask = in.width == 64 ? ~0ull : 0xFFFFFFFFull;
    uint64_t r = 0;
    switch (in.op) {
      case OP_ADD: r = (a + b) & mask; break;
      case OP_SUB: r = (a - b) & mask; break;
      case OP_MUL_LO: r = (a * b) & mask; break;
      case OP_MAD_LO: r = (a * b + c) & mask; break;
      case OP_MUL_WIDE:
        if (in.is_signed) r = (uint64_t)((int64_t)(int32_t)(uint32_t)a * (int64_t)(int32_t)(uint32_t)b);
        else r = (uint64_t)(uint32_t)a * (uint64_t)(uint32_t)b;
        break;
      case OP_FADD: r = canon(u2f((uint32_t)a) + u2f((uint32_t)b)); break;
      case OP_FSUB: r = canon(u2f((uint32_t)a) - u2f((uint32_t)b)); break;
      case OP_FMUL: r = canon(u2f((uint32_t)a) * u2f((uint32_t)b)); break;
      case OP_FFMA: r = canon(std::fma(u2f((uint32_t)a), u2f((uint32_t)b), u2f((uint32_t)c))); break;
      case OP_SETP:
        w.preds[(size_t)in.dst.reg * 32 + l] = compare(in, a, b) ? 1 : 0;
        return;
      case OP_SELP: r = c ? a : b; break;
      case OP_MOV: r = a & mask; break;
      default: break;
    }
    w.vals[(size_t)in.dst.reg * 32 + l] = r;
  }

  // What the analyser found for one warp access (all 0 when no lane passes the guard).
  struct MemInfo {
    uint32_t sectors = 0, lines = 0, degree = 0, faults = 0;
    bool cached = false;         // cache model: the access looked up a cache level
    uint32_t cache_latency = 0;  // ... and that level's latency (any table value, 0 included)
  };

  MemInfo memory_access(Warp& w, const Inst& in, uint32_t g, uint64_t block_linear,
                        std::vector<uint8_t>& shared, RaceLog* shared_races) {
    MemInfo mi;
    bool global = in.op == OP_LD_GLOBAL || in.op == OP_ST_GLOBAL;
    bool load = in.op == OP_LD_GLOBAL || in.op == OP_LD_SHARED;
    uint8_t* base = global ? gmem : shared.data();
    uint64_t size = global ? gmem_bytes : (uint64_t)shared.size();
    uint64_t addr[32];
    for (int l = 0; l < 32; ++l) {
      if (!((g >> l) & 1)) continue;
      uint64_t b = w.vals[(size_t)in.addr_reg * 32 + l];
      if (in.addr_width == 32) b &= 0xFFFFFFFFull;
      addr[l] = b + (uint64_t)in.addr_off;
    }
    if (g == 0) return mi;  // nothing to access or analyse
    // Analyse.
    if (global) {
      std::set<uint64_t> sectors, lines;
      for (int l = 0; l < 32; ++l) {
        if (!((g >> l) & 1)) continue;
        uint64_t first = addr[l], last = addr[l] + (uint64_t)(in.size - 1);
        sectors.insert(first >> 5);
        sectors.insert(last >> 5);
        lines.insert(first >> 7);
        lines.insert(last >> 7);
      }
      mi.sectors = (uint32_t)sectors.size();
      mi.lines = (uint32_t)lines.size();
      if (cfg->flags & ORACLE_FLAG_CACHE) {
        // the representative address: the lowest guard lane whose access is valid
        for (int l = 0; l < 32; ++l) {
          if (!((g >> l) & 1) || !valid(addr[l], size, in.size)) continue;
          const uint64_t line = addr[l] / 128;
          int level = 2;
          if (cache_access(w.l1, line)) level = 0;
          else if (cache_access(w.l2, line)) level = 1;
          w.cache_count[level]++;
          mi.cached = true;
          mi.cache_latency = lat(level == 0 ? ORACLE_LAT_L1_HIT : level == 1 ? ORACLE_LAT_L2_HIT : ORACLE_LAT_DRAM);
          break;
        }
      }
      if (load) {
        w.c.gld_n++;
        w.c.gld_sectors += (uint32_t)sectors.size();
        w.c.gld_lines += (uint32_t)lines.size();
      } else {
        w.c.gst_n++;
        w.c.gst_sectors += (uint32_t)sectors.size();
        w.c.gst_lines += (uint32_t)lines.size();
      }
    } else {
      uint32_t degree = 1;
      for (uint32_t bank = 0; bank < 32; ++bank) {
        uint32_t count = 0;
        bool same = true;
        uint64_t first = 0;
        for (int l = 0; l < 32; ++l) {
          if (!((g >> l) & 1)) continue;
          if (((addr[l] >> 2) & 31) != bank) continue;
          if (count == 0) first = addr[l];
          else if (addr[l] != first) same = false;
          ++count;
        }
        if (count >= 2 && !same) degree = std::max(degree, count);
      }
      mi.degree = degree;
      w.c.sh_n++;
      w.c.sh_degree_sum += degree;
      w.c.sh_degree_max = std::max(w.c.sh_degree_max, degree);
    }
    // Access, lanes in ascending order.
    RaceLog* races = global ? global_races : shared_races;
    for (int l = 0; l < 32; ++l) {
      if (!((g >> l) & 1)) continue;
      uint64_t a = addr[l];
      bool ok = valid(a, size, in.size);
      uint64_t tid = block_linear * (uint64_t)threads_per_block + (uint64_t)w.index * 32 + (uint64_t)l;
      if (!ok) {
        mi.faults++;
        w.c.fault_n++;
        w.c.status |= ORACLE_ST_FAULT;
        if (load) w.vals[(size_t)in.dst.reg * 32 + l] = 0;
        continue;
      }
      if (load) {
        uint64_t v = 0;
        memcpy(&v, base + a, (size_t)in.size);
        w.vals[(size_t)in.dst.reg * 32 + l] = v;
        if (races)
          for (int k = 0; k < in.size; ++k)
            races->note(global ? "global" : "shared", a + k, tid, false, base[a + k], base[a + k]);
      } else {
        uint64_t v = w.vals[(size_t)in.src[0].reg * 32 + l];
        if (races) {
          uint8_t bytes[8];
          memcpy(bytes, &v, 8);
          for (int k = 0; k < in.size; ++k)
            races->note(global ? "global" : "shared", a + k, tid, true, bytes[k], base[a + k]);
        }
        memcpy(base + a, &v, (size_t)in.size);
      }
    }
    return mi;
  }
};

void default_latency(uint16_t* lat) {
  for (int i = 0; i < ORACLE_NLAT; ++i) lat[i] = 0;
  // sm_80 values of the KernelScope latency model; classes the page does not list
  // (mad/mul.wide/setp/selp/mov, ld.param, ret) take 4 cycles like the integer and
  // control entries, ld.param like the constant-bank load.
  lat[ORACLE_LAT_INT32] = 4;
  lat[ORACLE_LAT_INT64] = 4;
  lat[ORACLE_LAT_FP32] = 4;
  lat[ORACLE_LAT_SETP] = 4;
  lat[ORACLE_LAT_SELP] = 4;
  lat[ORACLE_LAT_MOV] = 4;
  lat[ORACLE_LAT_LD_PARAM] = 4;
  lat[ORACLE_LAT_LD_GLOBAL] = 200;
  lat[ORACLE_LAT_LD_SHARED] = 23;
  lat[ORACLE_LAT_ST_GLOBAL] = 200;
  lat[ORACLE_LAT_ST_SHARED] = 23;
  lat[ORACLE_LAT_BRA] = 4;
  lat[ORACLE_LAT_BAR] = 20;
  lat[ORACLE_LAT_RET] = 4;
  // cache model (KernelScope memory-analysis part, cache parameters)
  lat[ORACLE_LAT_L1_HIT] = 28;
  lat[ORACLE_LAT_L2_HIT] = 150;
  lat[ORACLE_LAT_DRAM] = 400;
}

}  // namespace

extern "C" {

void oracle_default_latency(uint16_t out[ORACLE_NLAT]) { default_latency(out); }

int oracle_program_info(const char* ptx, size_t len, const char* entry, oracle_info* out, char* err,
                        size_t err_len) {
  try {
    Program p = load(ptx, len, entry);
    out->n_instrs = (uint32_t)p.code.size();
    out->n_params = (uint32_t)p.params.size();
    out->param_bytes = p.param_bytes;
    out->shared_bytes = p.shared_bytes;
    out->reg_words = p.reg_words;
    out->n_preds = (uint32_t)p.n_preds;
    return ORACLE_OK;
  } catch (const OracleError& e) {
    set_err(err, err_len, e.msg);
    return e.code;
  }
}

int oracle_param(const char* ptx, size_t len, const char* entry, uint32_t index, uint32_t* offset,
                 uint32_t* size, char* name, size_t name_len, char* err, size_t err_len) {
  try {
    Program p = load(ptx, len, entry);
    if (index >= p.params.size()) fail(ORACLE_E_INVALID_ARG, 0, "parameter index out of range");
    *offset = p.params[index].offset;
    *size = p.params[index].size;
    set_err(name, name_len, p.params[index].name);
    return ORACLE_OK;
  } catch (const OracleError& e) {
    set_err(err, err_len, e.msg);
    return e.code;
  }
}

int oracle_ipdom_table(const char* ptx, size_t len, const char* entry, uint32_t* out, uint32_t out_len,
                       char* err, size_t err_len) {
  try {
    Program p = load(ptx, len, entry);
    uint32_t n = (uint32_t)p.code.size();
    for (uint32_t i = 0; i < out_len && i < n; ++i) {
      const Inst& in = p.code[i];
      bool cond_branch = in.op == OP_BRA && in.has_guard;
      out[i] = cond_branch ? (p.rpc[i] == EXIT_PC ? n : p.rpc[i]) : 0xFFFFFFFFu;
    }
    return ORACLE_OK;
  } catch (const OracleError& e) {
    set_err(err, err_len, e.msg);
    return e.code;
  }
}

int oracle_run(const char* ptx, size_t len, const char* entry, const oracle_cfg* cfg, const void* params,
               size_t params_len, uint8_t* gmem, uint8_t* counters, uint8_t* trace, char* err, size_t err_len) {
  try {
    Program p = load(ptx, len, entry);
    for (int k = 0; k < 3; ++k)
      if (cfg->grid[k] == 0 || cfg->block[k] == 0) fail(ORACLE_E_INVALID_ARG, 0, "zero grid or block dimension");
    uint64_t tpb = (uint64_t)cfg->block[0] * cfg->block[1] * cfg->block[2];
    if (tpb > 1024) fail(ORACLE_E_INVALID_ARG, 0, "more than 1024 threads per block");
    if (params_len < p.param_bytes) fail(ORACLE_E_INVALID_ARG, 0, "parameter buffer too short");
    if ((cfg->flags & ORACLE_FLAG_CACHE) && !cfg->cache) fail(ORACLE_E_INVALID_ARG, 0, "cache model without an output buffer");
    if ((cfg->flags & ORACLE_FLAG_CACHE) && cfg->gmem_bytes > (1ull << 38))
      fail(ORACLE_E_UNSUPPORTED, 0, "cache model over more than 2^38 bytes of memory");
    uint64_t n_blocks = (uint64_t)cfg->grid[0] * cfg->grid[1] * cfg->grid[2];
    std::vector<uint64_t> blocks;
    if (cfg->n_block_list) {
      for (uint64_t i = 0; i < cfg->n_block_list; ++i) {
        if (cfg->block_list[i] >= n_blocks) fail(ORACLE_E_INVALID_ARG, 0, "block id out of range");
        blocks.push_back(cfg->block_list[i]);
      }
    } else {
      for (uint64_t b = 0; b < n_blocks; ++b) blocks.push_back(b);
    }
    Sim sim;
    sim.p = &p;
    sim.cfg = cfg;
    sim.params = (const uint8_t*)params;
    sim.gmem = gmem;
    sim.gmem_bytes = cfg->gmem_bytes;
    sim.threads_per_block = (uint32_t)tpb;
    sim.warps_per_block = (uint32_t)((tpb + 31) / 32);
    size_t slot = 16 + ((cfg->flags & ORACLE_FLAG_EXT_TRACE) ? 16 : 8) * (size_t)cfg->trace_cap;
    RaceLog races;
    bool check = (cfg->flags & ORACLE_FLAG_CHECK_RACES) != 0;
    if (check) sim.global_races = &races;
    unsigned nt = cfg->n_threads ? cfg->n_threads : std::max(1u, std::thread::hardware_concurrency());
    if (check) nt = 1;
    nt = (unsigned)std::min<uint64_t>(nt, blocks.size() ? blocks.size() : 1);
    std::vector<std::string> errors(nt);
    std::vector<int> codes(nt, 0);
    auto worker = [&](unsigned id) {
      // Round to nearest even, no flush-to-zero, no denormals-are-zero.
      _mm_setcsr(0x1F80);
      uint64_t lo = blocks.size() * id / nt, hi = blocks.size() * (id + 1) / nt;
      try {
        for (uint64_t i = lo; i < hi; ++i) {
          oracle_counters* c = (oracle_counters*)(counters + sizeof(oracle_counters) * sim.warps_per_block * i);
          uint8_t* cw = cfg->cache ? cfg->cache + (size_t)ORACLE_CACHE_WARP_BYTES * sim.warps_per_block * i : nullptr;
          sim.run_block(blocks[i], c, trace + slot * sim.warps_per_block * i, cw);
        }
      } catch (const OracleError& e) {
        codes[id] = e.code;
        errors[id] = e.msg;
      }
    };
    if (nt == 1) {
      unsigned csr = _mm_getcsr();
      worker(0);
      _mm_setcsr(csr);
    } else {
      std::vector<std::thread> ts;
      for (unsigned id = 0; id < nt; ++id) ts.emplace_back(worker, id);
      for (auto& t : ts) t.join();
    }
    for (unsigned id = 0; id < nt; ++id)
      if (codes[id]) fail(codes[id], 0, "%s", errors[id].c_str());
    if (check && races.raced) {
      set_err(err, err_len, races.first);
      return ORACLE_E_RACE;
    }
    return ORACLE_OK;
  } catch (const OracleError& e) {
    set_err(err, err_len, e.msg);
    return e.code;
  }
}

}  // extern "C"
