// ks_host.cpp -- host side of libkscope: PTX-subset front end, post-dominator
// reconvergence points, decoded-table encoder and the C ABI entry points.
//
// The grammar follows the PTX-parser part of the KernelScope backend
// documentation (github.com/briefgaming/kernelscope): module directives, a
// .visible .entry with .param declarations, .reg declarations "%name<N>" that
// declare N registers numbered from 0, and instructions made of an optional
// "@" / "@!" predicate guard, an opcode with dotted modifiers and a comma
// separated operand list.  Reconvergence at the immediate post-dominator of a
// divergent branch is the SIMT-stack entry (pc, mask, reconvergence pc) of the
// execution-simulator part of the same page.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/ks.h"
#include "ks_isa.h"
#include "ks_launch.h"

using namespace ks;

// ---------------------------------------------------------------------------- errors

static thread_local std::string g_last_error;

namespace {

struct KsFail {
  ks_status code;
};

[[noreturn]] void raise(ks_status code, int line, const char* fmt, ...) {
  char buf[400];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = line > 0 ? "line " + std::to_string(line) + ": " + buf : std::string(buf);
  throw KsFail{code};
}

// ---------------------------------------------------------------------------- lexer

enum TokKind { T_WORD, T_NUM, T_PUNCT, T_END };

struct Tok {
  TokKind kind;
  std::string text;
  int line;
  bool glued = false;  // follows the previous token with no space or comment between
};

bool word_start(char c) {
  return (c >= 'a' && c <= 'z') || (c >= 'A' && c <= 'Z') || c == '_' || c == '$' || c == '%' || c == '.';
}
bool word_char(char c) {
  return word_start(c) || (c >= '0' && c <= '9');
}

// A label: a letter, '_' or '$', then letters, digits, '_' or '$' (no dots).
bool label_name(const std::string& w) {
  if (w.empty() || !((w[0] >= 'a' && w[0] <= 'z') || (w[0] >= 'A' && w[0] <= 'Z') || w[0] == '_' || w[0] == '$'))
    return false;
  for (char c : w)
    if (!(word_char(c) && c != '.' && c != '%')) return false;
  return true;
}

// Splits the text into words (identifiers with their dots: "ld.global.f32",
// "%tid.x", ".reg"), numbers and single-character punctuation.  Line-scoped
// directives (.loc/.file and the module header directives) are handled here.
std::vector<Tok> lex(const char* src, size_t len) {
  std::vector<Tok> out;
  int line = 1;
  size_t i = 0;
  auto skip_line = [&]() {
    while (i < len && src[i] != '\n') ++i;
  };
  bool line_start = true;
  size_t prev_end = (size_t)-1;  // end of the previous token
  auto push = [&](TokKind k, std::string text, size_t at, size_t end) {
    out.push_back({k, std::move(text), line, at == prev_end});
    prev_end = end;
  };
  // The rest of a line-scoped directive: up to the end of its line with comments
  // removed.  A block comment that spans lines ends the directive at its first
  // newline; the text after the comment is on a later line and lexed as usual.
  auto skip_directive_rest = [&]() {
    while (i < len && src[i] != '\n') {
      if (src[i] == '/' && i + 1 < len && src[i + 1] == '/') {
        skip_line();
        return;
      }
      if (src[i] == '/' && i + 1 < len && src[i + 1] == '*') {
        size_t k = i + 2;
        bool spans = false;
        while (k + 1 < len && !(src[k] == '*' && src[k + 1] == '/')) {
          if (src[k] == '\n') {
            ++line;
            spans = true;
          }
          ++k;
        }
        if (k + 1 >= len) raise(KS_E_PARSE, line, "unterminated comment");
        i = k + 2;
        if (spans) {
          line_start = true;
          return;
        }
        continue;
      }
      ++i;
    }
  };
  while (i < len) {
    char c = src[i];
    if (c == '\n') {
      ++line;
      ++i;
      line_start = true;
      continue;
    }
    if (c == ' ' || c == '\t' || c == '\r') {
      ++i;
      continue;
    }
    if (c == '/' && i + 1 < len && src[i + 1] == '/') {
      skip_line();
      continue;
    }
    if (c == '/' && i + 1 < len && src[i + 1] == '*') {
      i += 2;
      while (i + 1 < len && !(src[i] == '*' && src[i + 1] == '/')) {
        if (src[i] == '\n') {
          ++line;
          line_start = true;  // what follows the comment starts its line
        }
        ++i;
      }
      if (i + 1 >= len) raise(KS_E_PARSE, line, "unterminated comment");
      i += 2;
      continue;
    }
    bool at_line_start = line_start;
    line_start = false;
    if (word_start(c)) {
      size_t j = i;
      while (j < len && word_char(src[j])) ++j;
      std::string w(src + i, j - i);
      if (at_line_start && (w == ".loc" || w == ".file" || w == ".section")) {
        i = j;  // source-map directives are ignored
        skip_directive_rest();
        continue;
      }
      if (w == ".version" || w == ".target" || w == ".address_size") {
        // module header directive: the rest of its line is its argument (not used)
        push(T_WORD, w, i, j);
        i = j;
        const size_t k = i;
        skip_directive_rest();
        push(T_WORD, std::string(src + k, i - k), k, i);
        push(T_PUNCT, ";", i, i);
        continue;
      }
      push(T_WORD, w, i, j);
      i = j;
      continue;
    }
    if (c >= '0' && c <= '9') {
      size_t j = i;
      while (j < len && (word_char(src[j]))) ++j;
      push(T_NUM, std::string(src + i, j - i), i, j);
      i = j;
      continue;
    }
    if (strchr(",;:[](){}+-@!<>", c)) {
      push(T_PUNCT, std::string(1, c), i, i + 1);
      ++i;
      continue;
    }
    raise(KS_E_PARSE, line, "unexpected character '%c'", c);
  }
  out.push_back({T_END, "", line, false});
  return out;
}

// ---------------------------------------------------------------------------- program model

struct RegInfo {
  int width;   // 32, 64 or 1 (predicate)
  int slot;    // first 32-bit slot (value registers) or predicate index
  int sb;      // scoreboard index
};

struct Operand {
  uint8_t kind = KK_NONE;
  uint8_t slot = 0;     // register slot / special id / predicate
  uint8_t sb = KS_NO_SB;
  uint64_t imm = 0;
};

struct ParamInfo {
  std::string name;
  uint32_t offset, size;
};

struct Decoded {
  KsInst in;
  int line;
  std::string target_label;
  bool is_branch = false, is_ret = false, guarded = false;
};

}  // namespace

struct ks_program {
  std::vector<Decoded> code;
  std::vector<ParamInfo> params;
  uint32_t param_bytes = 0;
  uint32_t shared_bytes = 0;
  uint32_t reg_slots = 0;
  uint32_t n_preds = 0;
  std::vector<uint32_t> rpc;   // per instruction: reconvergence index, n_instrs = exit
};

namespace {

struct TypeDesc {
  int width;
  bool is_signed, is_float, bits;
};

bool type_desc(const std::string& t, TypeDesc& d) {
  static const std::map<std::string, TypeDesc> table = {
      {"s32", {32, true, false, false}}, {"u32", {32, false, false, false}}, {"b32", {32, false, false, true}},
      {"f32", {32, false, true, false}}, {"s64", {64, true, false, false}}, {"u64", {64, false, false, false}},
      {"b64", {64, false, false, true}}, {"pred", {1, false, false, false}}};
  auto it = table.find(t);
  if (it == table.end()) return false;
  d = it->second;
  return true;
}

std::vector<std::string> dotted(const std::string& w) {
  std::vector<std::string> parts;
  size_t s = 0;
  for (size_t k = 0; k <= w.size(); ++k) {
    if (k == w.size() || w[k] == '.') {
      parts.push_back(w.substr(s, k - s));
      s = k + 1;
    }
  }
  return parts;
}

bool parse_u64(const std::string& s, uint64_t& v) {
  if (s.empty()) return false;
  uint64_t x = 0;
  if (s.size() > 2 && s[0] == '0' && (s[1] == 'x' || s[1] == 'X')) {
    if (s.size() > 18) return false;
    for (size_t k = 2; k < s.size(); ++k) {
      char c = s[k];
      int d = (c >= '0' && c <= '9') ? c - '0' : (c >= 'a' && c <= 'f') ? c - 'a' + 10 : (c >= 'A' && c <= 'F') ? c - 'A' + 10 : -1;
      if (d < 0) return false;
      x = (x << 4) | (uint64_t)d;
    }
  } else {
    for (char c : s) {
      if (c < '0' || c > '9') return false;
      if (x > (UINT64_MAX - 9) / 10) return false;
      x = x * 10 + (uint64_t)(c - '0');
    }
  }
  v = x;
  return true;
}

class Front {
 public:
  Front(const std::vector<Tok>& t) : toks(t) {}

  ks_program* run(const char* entry) {
    std::unique_ptr<ks_program> prog(new ks_program());
    P = prog.get();
    bool found = false;
    while (peek().kind != T_END) {
      const Tok& t = peek();
      if (t.kind == T_WORD && (t.text == ".version" || t.text == ".target" || t.text == ".address_size")) {
        pos += 3;  // directive, argument, ';'
        continue;
      }
      bool visible = false;
      if (is_word(".visible")) {
        ++pos;
        visible = true;
      }
      (void)visible;
      if (!is_word(".entry")) raise(KS_E_UNSUPPORTED, t.line, "unsupported module-level statement '%s'", t.text.c_str());
      ++pos;
      std::string name = expect_word("entry name").text;
      bool take = !found && (entry == nullptr || entry[0] == 0 || name == entry);
      if (take) {
        found = true;
        entry_body();
      } else {
        skip_entry();
      }
    }
    if (!found) raise(KS_E_PARSE, 0, entry && entry[0] ? "entry '%s' not found" : "no .entry in module", entry ? entry : "");
    resolve_labels();
    if (P->code.size() > KS_MAX_INSTRS) raise(KS_E_UNSUPPORTED, 0, "program has more than %d instructions", KS_MAX_INSTRS);
    prog.release();
    return P;
  }

 private:
  const std::vector<Tok>& toks;
  size_t pos = 0;
  ks_program* P = nullptr;
  std::unordered_map<std::string, RegInfo> regs;
  std::unordered_map<std::string, uint32_t> shared_vars;
  std::unordered_map<std::string, int> labels;
  int n_vals = 0;

  const Tok& peek(size_t k = 0) const { return toks[std::min(pos + k, toks.size() - 1)]; }
  bool is_punct(const char* p) const { return peek().kind == T_PUNCT && peek().text == p; }
  bool is_word(const char* w) const { return peek().kind == T_WORD && peek().text == w; }
  const Tok& expect_word(const char* what) {
    if (peek().kind != T_WORD) raise(KS_E_PARSE, peek().line, "expected %s, got '%s'", what, peek().text.c_str());
    return toks[pos++];
  }
  void expect_punct(const char* p) {
    if (!is_punct(p)) raise(KS_E_PARSE, peek().line, "expected '%s', got '%s'", p, peek().text.c_str());
    ++pos;
  }

  void skip_entry() {
    int depth = 0;
    while (peek().kind != T_END) {
      if (is_punct("{")) ++depth;
      if (is_punct("}")) {
        --depth;
        if (depth == 0) {
          ++pos;
          return;
        }
      }
      ++pos;
    }
    raise(KS_E_PARSE, peek().line, "unterminated entry");
  }

  void entry_body() {
    // parameter list
    uint32_t off = 0;
    if (is_punct("(")) {
      ++pos;
      while (!is_punct(")")) {
        const Tok& d = expect_word(".param");
        if (d.text != ".param") raise(KS_E_PARSE, d.line, "expected .param");
        const Tok& ty = expect_word("parameter type");
        TypeDesc td;
        if (ty.text.size() < 2 || !type_desc(ty.text.substr(1), td) || td.width == 1)
          raise(KS_E_UNSUPPORTED, ty.line, "unsupported parameter type '%s'", ty.text.c_str());
        const Tok& nt = expect_word("parameter name");
        const std::string nm = nt.text;
        uint32_t size = (uint32_t)td.width / 8;
        off = (off + size - 1) / size * size;
        P->params.push_back({nm, off, size});
        off += size;
        if (!is_punct(")")) {
          if (!is_punct(",")) raise(KS_E_PARSE, nt.line, "expected ',' after parameter %s, got '%s'", nm.c_str(), peek().text.c_str());
          ++pos;
        }
      }
      ++pos;
    }
    P->param_bytes = off;
    if (off > KS_MAX_PARAM_BYTES) raise(KS_E_UNSUPPORTED, peek().line, "parameter block larger than %d bytes", KS_MAX_PARAM_BYTES);
    expect_punct("{");
    while (!is_punct("}")) {
      if (peek().kind == T_END) raise(KS_E_PARSE, peek().line, "unterminated entry body");
      statement();
    }
    ++pos;
  }

  void statement() {
    const Tok& t = peek();
    if (t.kind == T_PUNCT && t.text == "{") raise(KS_E_UNSUPPORTED, t.line, "nested blocks are not supported");
    if (t.kind == T_WORD && peek(1).kind == T_PUNCT && peek(1).text == ":") {
      if (!label_name(t.text)) raise(KS_E_PARSE, t.line, "bad label name '%s'", t.text.c_str());
      if (!peek(1).glued) raise(KS_E_PARSE, t.line, "space between label '%s' and its ':'", t.text.c_str());
      if (labels.count(t.text)) raise(KS_E_PARSE, t.line, "label '%s' defined twice", t.text.c_str());
      labels[t.text] = (int)P->code.size();
      pos += 2;
      return;
    }
    if (t.kind == T_WORD && t.text == ".reg") {
      reg_decl();
      return;
    }
    if (t.kind == T_WORD && t.text == ".shared") {
      shared_decl();
      return;
    }
    if (t.kind == T_WORD && t.text[0] == '.') raise(KS_E_UNSUPPORTED, t.line, "unsupported directive '%s'", t.text.c_str());
    instruction();
  }

  void declare(int line, const std::string& name, const TypeDesc& td) {
    if (regs.count(name)) raise(KS_E_PARSE, line, "register '%s' declared twice", name.c_str());
    RegInfo r;
    r.width = td.width;
    if (td.width == 1) {
      r.slot = (int)P->n_preds++;
      r.sb = (int)KS_SB_PRED_BASE + r.slot;
    } else {
      r.slot = (int)P->reg_slots;
      r.sb = n_vals++;
      P->reg_slots += (uint32_t)td.width / 32;
    }
    regs[name] = r;
  }

  void reg_decl() {
    int line = peek().line;
    ++pos;
    const Tok& ty = expect_word("register type");
    TypeDesc td;
    if (ty.text.size() < 2 || !type_desc(ty.text.substr(1), td)) raise(KS_E_UNSUPPORTED, ty.line, "unsupported register type '%s'", ty.text.c_str());
    while (true) {
      std::string nm = expect_word("register name").text;
      if (is_punct("<")) {
        if (!peek().glued) raise(KS_E_PARSE, line, "space between register name '%s' and its count", nm.c_str());
        ++pos;
        uint64_t n;
        if (peek().kind != T_NUM || !parse_u64(peek().text, n) || n == 0 || n > 4096) raise(KS_E_PARSE, line, "bad register count");
        ++pos;
        expect_punct(">");
        for (uint64_t k = 0; k < n; ++k) declare(line, nm + std::to_string(k), td);
      } else {
        declare(line, nm, td);
      }
      if (is_punct(",")) {
        ++pos;
        continue;
      }
      break;
    }
    expect_punct(";");
  }

  void shared_decl() {
    int line = peek().line;
    ++pos;
    uint64_t align = 0;
    if (is_word(".align")) {
      ++pos;
      if (peek().kind != T_NUM || !parse_u64(peek().text, align) || align == 0 || (align & (align - 1)))
        raise(KS_E_PARSE, line, "bad .align");
      ++pos;
    }
    const Tok& ty = expect_word("element type");
    static const std::map<std::string, uint32_t> esz = {{".b8", 1}, {".u8", 1}, {".s8", 1}, {".b16", 2}, {".u16", 2},
                                                         {".s16", 2}, {".b32", 4}, {".u32", 4}, {".s32", 4}, {".f32", 4},
                                                         {".b64", 8}, {".u64", 8}, {".s64", 8}};
    auto it = esz.find(ty.text);
    if (it == esz.end()) raise(KS_E_UNSUPPORTED, line, "unsupported .shared type '%s'", ty.text.c_str());
    std::string nm = expect_word("shared variable name").text;
    uint64_t count = 1;
    if (is_punct("[")) {
      ++pos;
      if (peek().kind != T_NUM || !parse_u64(peek().text, count)) raise(KS_E_PARSE, line, "bad array size");
      ++pos;
      expect_punct("]");
    }
    if (!align) align = it->second;
    uint64_t off = (P->shared_bytes + align - 1) / align * align;
    uint64_t end = off + count * it->second;
    if (end > KS_MAX_SHARED_BYTES) raise(KS_E_UNSUPPORTED, line, "shared window larger than %d bytes", KS_MAX_SHARED_BYTES);
    shared_vars[nm] = (uint32_t)off;
    P->shared_bytes = (uint32_t)end;
    expect_punct(";");
  }

  // ---- operands

  struct RawOperand {
    enum { WORD, NUM, MEM } kind;
    std::string text;      // WORD/NUM text, MEM base
    bool neg = false;      // leading '-' on a number
    int64_t mem_off = 0;
    int line;
  };

  RawOperand raw_operand() {
    RawOperand r;
    r.line = peek().line;
    if (is_punct("[")) {
      ++pos;
      r.kind = RawOperand::MEM;
      r.text = expect_word("address base").text;
      if (is_punct("+") || is_punct("-")) {
        bool minus = is_punct("-");
        ++pos;
        if (is_punct("-")) {  // "+-imm"
          minus = !minus;
          ++pos;
          if (!peek().glued) raise(KS_E_PARSE, r.line, "space between '-' and its number");
        }
        uint64_t v;
        if (peek().kind != T_NUM || !parse_u64(peek().text, v) || v > (1ull << 62)) raise(KS_E_PARSE, r.line, "bad address offset");
        ++pos;
        r.mem_off = minus ? -(int64_t)v : (int64_t)v;
      }
      expect_punct("]");
      return r;
    }
    if (is_punct("-")) {
      ++pos;
      r.neg = true;
      if (!peek().glued) raise(KS_E_PARSE, r.line, "space between '-' and its number");
    }
    if (peek().kind == T_NUM) {
      r.kind = RawOperand::NUM;
      r.text = toks[pos++].text;
      return r;
    }
    if (r.neg) raise(KS_E_PARSE, r.line, "'-' must precede a number");
    r.kind = RawOperand::WORD;
    r.text = expect_word("operand").text;
    return r;
  }

  std::vector<RawOperand> operand_list() {
    std::vector<RawOperand> v;
    if (is_punct(";")) return v;
    while (true) {
      v.push_back(raw_operand());
      if (is_punct(",")) {
        ++pos;
        continue;
      }
      break;
    }
    return v;
  }

  const RegInfo& reg_of(const RawOperand& r) {
    if (r.kind != RawOperand::WORD) raise(KS_E_PARSE, r.line, "expected a register");
    auto it = regs.find(r.text);
    if (it == regs.end()) raise(KS_E_PARSE, r.line, "undeclared register %s", r.text.c_str());
    return it->second;
  }

  Operand value_src(const RawOperand& r, int width, bool is_float, bool allow_special) {
    Operand o;
    if (r.kind == RawOperand::WORD) {
      auto it = regs.find(r.text);
      if (it != regs.end()) {
        if (it->second.width == 1) raise(KS_E_PARSE, r.line, "predicate %s used as a value", r.text.c_str());
        if (it->second.width != width) raise(KS_E_PARSE, r.line, "register %s is %d-bit, operand is %d-bit", r.text.c_str(), it->second.width, width);
        o.kind = KK_REG;
        o.slot = (uint8_t)it->second.slot;
        o.sb = (uint8_t)it->second.sb;
        return o;
      }
      static const char* sp[] = {"%tid.x", "%tid.y", "%tid.z", "%ntid.x", "%ntid.y", "%ntid.z", "%ctaid.x",
                                 "%ctaid.y", "%ctaid.z", "%nctaid.x", "%nctaid.y", "%nctaid.z", "%laneid"};
      for (int k = 0; k < 13; ++k) {
        if (r.text == sp[k]) {
          if (!allow_special) raise(KS_E_UNSUPPORTED, r.line, "special register %s only allowed as a mov source", r.text.c_str());
          if (width != 32) raise(KS_E_PARSE, r.line, "special registers are 32-bit");
          o.kind = KK_SPECIAL;
          o.slot = (uint8_t)k;
          return o;
        }
      }
      auto sv = shared_vars.find(r.text);
      if (sv != shared_vars.end() && allow_special && !is_float) {
        o.kind = KK_IMM;
        o.imm = sv->second;
        return o;
      }
      if (r.text[0] == '%') raise(KS_E_PARSE, r.line, "undeclared register %s", r.text.c_str());
      raise(KS_E_PARSE, r.line, "bad operand '%s'", r.text.c_str());
    }
    if (r.kind == RawOperand::NUM) {
      const std::string& s = r.text;
      if (s.size() == 10 && s[0] == '0' && (s[1] == 'f' || s[1] == 'F') && !r.neg) {
        uint64_t bits;
        if (!parse_u64("0x" + s.substr(2), bits)) raise(KS_E_PARSE, r.line, "bad f32 literal '%s'", s.c_str());
        if (width != 32) raise(KS_E_PARSE, r.line, "0f literal in a 64-bit operand");
        o.kind = KK_IMM;
        o.imm = bits;
        return o;
      }
      if (is_float) raise(KS_E_UNSUPPORTED, r.line, "f32 immediates must be 0fXXXXXXXX bit patterns");
      uint64_t v;
      if (!parse_u64(s, v)) raise(KS_E_PARSE, r.line, "bad integer literal '%s'", s.c_str());
      if (width == 32) {
        if (r.neg ? v > 0x80000000ull : v > 0xFFFFFFFFull) raise(KS_E_PARSE, r.line, "immediate does not fit 32 bits");
      }
      if (r.neg) v = 0 - v;
      o.kind = KK_IMM;
      o.imm = width == 32 ? (v & 0xFFFFFFFFull) : v;
      return o;
    }
    raise(KS_E_PARSE, r.line, "unexpected memory operand");
  }

  void set_src(KsInst& in, int k, const Operand& o) {
    in.src[k] = o.slot;
    in.kinds = (uint8_t)(in.kinds | (o.kind << (2 * k)));
    in.sb[k] = o.sb;
    if (o.kind == KK_IMM) in.imm[k] = o.imm;
  }

  void set_dst_reg(KsInst& in, const RawOperand& r, int width) {
    const RegInfo& ri = reg_of(r);
    if (ri.width == 1) raise(KS_E_PARSE, r.line, "predicate %s used as a value", r.text.c_str());
    if (ri.width != width) raise(KS_E_PARSE, r.line, "register %s is %d-bit, operand is %d-bit", r.text.c_str(), ri.width, width);
    in.dst = (uint8_t)ri.slot;
    in.sb_dst = (uint8_t)ri.sb;
  }

  uint8_t pred_index(const RawOperand& r, uint8_t* sb) {
    const RegInfo& ri = reg_of(r);
    if (ri.width != 1) raise(KS_E_PARSE, r.line, "expected a predicate, got %s", r.text.c_str());
    if (sb) *sb = (uint8_t)ri.sb;
    return (uint8_t)ri.slot;
  }

  void instruction() {
    Decoded d;
    memset(&d.in, 0, sizeof d.in);
    KsInst& in = d.in;
    for (int k = 0; k < 4; ++k) in.sb[k] = KS_NO_SB;
    in.sb_dst = KS_NO_SB;
    in.rpc = KS_RPC_EXIT;
    d.line = peek().line;
    if (is_punct("@")) {
      ++pos;
      bool neg = false;
      if (is_punct("!")) {
        if (!peek().glued) raise(KS_E_PARSE, peek().line, "space inside the guard");
        ++pos;
        neg = true;
      }
      if (!peek().glued) raise(KS_E_PARSE, peek().line, "space inside the guard");
      RawOperand g;
      g.kind = RawOperand::WORD;
      g.line = peek().line;
      g.text = expect_word("guard predicate").text;
      in.guard = pred_index(g, &in.sb[3]);
      in.flags |= KF_GUARD | (neg ? KF_GUARD_NEG : 0);
      d.guarded = true;
    }
    const Tok& opt = expect_word("instruction");
    std::vector<std::string> m = dotted(opt.text);
    if (!is_punct(";") && peek().glued) raise(KS_E_PARSE, opt.line, "expected a space after '%s'", opt.text.c_str());
    std::vector<RawOperand> ops = operand_list();
    expect_punct(";");
    const std::string& base = m[0];
    auto nops = [&](size_t n) {
      if (ops.size() != n) raise(KS_E_PARSE, d.line, "%s takes %zu operands", opt.text.c_str(), n);
    };
    auto bad_form = [&]() { raise(KS_E_UNSUPPORTED, d.line, "unsupported instruction '%s'", opt.text.c_str()); };
    auto tdesc = [&](const std::string& t) {
      TypeDesc td;
      if (!type_desc(t, td) || td.width == 1) bad_form();
      return td;
    };
    uint8_t lat_class = KS_LAT_INT32;

    if (base == "add" || base == "sub") {
      bool rn = m.size() == 3 && m[1] == "rn";
      if (!(m.size() == 2 || rn)) bad_form();
      TypeDesc td = tdesc(m.back());
      if (td.bits || (rn && !td.is_float)) bad_form();
      nops(3);
      bool add = base == "add";
      if (td.is_float) {
        in.op = add ? KO_FADD : KO_FSUB;
        lat_class = KS_LAT_FP32;
      } else if (td.width == 64) {
        in.op = add ? KO_ADD64 : KO_SUB64;
        lat_class = KS_LAT_INT64;
      } else {
        in.op = add ? KO_ADD32 : KO_SUB32;
      }
      set_dst_reg(in, ops[0], td.width);
      set_src(in, 0, value_src(ops[1], td.width, td.is_float, false));
      set_src(in, 1, value_src(ops[2], td.width, td.is_float, false));
    } else if (base == "mul") {
      if (m.size() == 3 && m[1] == "lo") {
        TypeDesc td = tdesc(m[2]);
        if (td.is_float || td.bits) bad_form();
        in.op = td.width == 64 ? KO_MUL64 : KO_MUL32;
        lat_class = td.width == 64 ? KS_LAT_INT64 : KS_LAT_INT32;
        nops(3);
        set_dst_reg(in, ops[0], td.width);
        set_src(in, 0, value_src(ops[1], td.width, false, false));
        set_src(in, 1, value_src(ops[2], td.width, false, false));
      } else if (m.size() == 3 && m[1] == "wide") {
        TypeDesc td = tdesc(m[2]);
        if (td.is_float || td.bits || td.width != 32) bad_form();
        in.op = td.is_signed ? KO_MULWIDE_S : KO_MULWIDE_U;
        nops(3);
        set_dst_reg(in, ops[0], 64);
        set_src(in, 0, value_src(ops[1], 32, false, false));
        set_src(in, 1, value_src(ops[2], 32, false, false));
      } else if ((m.size() == 2 && m[1] == "f32") || (m.size() == 3 && m[1] == "rn" && m[2] == "f32")) {
        in.op = KO_FMUL;
        lat_class = KS_LAT_FP32;
        nops(3);
        set_dst_reg(in, ops[0], 32);
        set_src(in, 0, value_src(ops[1], 32, true, false));
        set_src(in, 1, value_src(ops[2], 32, true, false));
      } else {
        bad_form();
      }
    } else if (base == "mad") {
      if (!(m.size() == 3 && m[1] == "lo")) bad_form();
      TypeDesc td = tdesc(m[2]);
      if (td.is_float || td.bits) bad_form();
      in.op = td.width == 64 ? KO_MAD64 : KO_MAD32;
      lat_class = td.width == 64 ? KS_LAT_INT64 : KS_LAT_INT32;
      nops(4);
      set_dst_reg(in, ops[0], td.width);
      for (int k = 0; k < 3; ++k) set_src(in, k, value_src(ops[k + 1], td.width, false, false));
    } else if (base == "fma") {
      if (!(m.size() == 3 && m[1] == "rn" && m[2] == "f32")) bad_form();
      in.op = KO_FFMA;
      lat_class = KS_LAT_FP32;
      nops(4);
      set_dst_reg(in, ops[0], 32);
      for (int k = 0; k < 3; ++k) set_src(in, k, value_src(ops[k + 1], 32, true, false));
    } else if (base == "setp") {
      if (m.size() != 3) bad_form();
      TypeDesc td = tdesc(m[2]);
      const std::string& c = m[1];
      bool uns = !td.is_signed && !td.is_float && !td.bits;
      static const std::map<std::string, uint8_t> cmps = {{"eq", KC_EQ}, {"ne", KC_NE}, {"lt", KC_LT}, {"le", KC_LE},
                                                          {"gt", KC_GT}, {"ge", KC_GE}, {"lo", KC_LT}, {"ls", KC_LE},
                                                          {"hi", KC_GT}, {"hs", KC_GE}};
      auto it = cmps.find(c);
      if (it == cmps.end()) bad_form();
      bool unsigned_only = c == "lo" || c == "ls" || c == "hi" || c == "hs";
      if (unsigned_only && !uns) bad_form();
      if (td.bits && !(c == "eq" || c == "ne")) bad_form();
      in.cmp = it->second;
      if (td.is_float) in.op = KO_SETP_F32;
      else if (td.width == 64) in.op = td.is_signed ? KO_SETP_S64 : KO_SETP_U64;
      else in.op = td.is_signed ? KO_SETP_S32 : KO_SETP_U32;
      lat_class = KS_LAT_SETP;
      nops(3);
      in.dst = pred_index(ops[0], &in.sb_dst);
      set_src(in, 0, value_src(ops[1], td.width, td.is_float, false));
      set_src(in, 1, value_src(ops[2], td.width, td.is_float, false));
    } else if (base == "selp") {
      if (m.size() != 2) bad_form();
      TypeDesc td = tdesc(m[1]);
      in.op = td.width == 64 ? KO_SELP64 : KO_SELP32;
      lat_class = KS_LAT_SELP;
      nops(4);
      set_dst_reg(in, ops[0], td.width);
      set_src(in, 0, value_src(ops[1], td.width, td.is_float, false));
      set_src(in, 1, value_src(ops[2], td.width, td.is_float, false));
      Operand p;
      p.kind = KK_REG;
      p.slot = pred_index(ops[3], &p.sb);
      set_src(in, 2, p);
    } else if (base == "mov") {
      if (m.size() != 2) bad_form();
      TypeDesc td = tdesc(m[1]);
      in.op = td.width == 64 ? KO_MOV64 : KO_MOV32;
      lat_class = KS_LAT_MOV;
      nops(2);
      set_dst_reg(in, ops[0], td.width);
      set_src(in, 0, value_src(ops[1], td.width, td.is_float, true));
    } else if (base == "ld" || base == "st") {
      if (m.size() != 3) bad_form();
      TypeDesc td = tdesc(m[2]);
      const std::string& space = m[1];
      nops(2);
      bool w64 = td.width == 64;
      if (base == "ld" && space == "param") {
        in.op = w64 ? KO_LDP64 : KO_LDP32;
        lat_class = KS_LAT_LD_PARAM;
        set_dst_reg(in, ops[0], td.width);
        const RawOperand& a = ops[1];
        if (a.kind != RawOperand::MEM) raise(KS_E_PARSE, a.line, "expected [param]");
        bool ok = false;
        for (const ParamInfo& p : P->params) {
          if (p.name == a.text) {
            if (a.mem_off < 0 || (uint64_t)a.mem_off + (uint64_t)td.width / 8 > p.size)
              raise(KS_E_PARSE, a.line, "access outside parameter %s", p.name.c_str());
            in.aux = (uint16_t)(p.offset + (uint32_t)a.mem_off);
            ok = true;
          }
        }
        if (!ok) raise(KS_E_PARSE, a.line, "unknown parameter %s", a.text.c_str());
      } else if (space == "global" || space == "shared") {
        bool g = space == "global";
        bool ld = base == "ld";
        if (ld) {
          in.op = g ? (w64 ? KO_LDG64 : KO_LDG32) : (w64 ? KO_LDS64 : KO_LDS32);
          lat_class = g ? KS_LAT_LD_GLOBAL : KS_LAT_LD_SHARED;
        } else {
          in.op = g ? (w64 ? KO_STG64 : KO_STG32) : (w64 ? KO_STS64 : KO_STS32);
          lat_class = g ? KS_LAT_ST_GLOBAL : KS_LAT_ST_SHARED;
        }
        const RawOperand& a = ld ? ops[1] : ops[0];
        if (a.kind != RawOperand::MEM) raise(KS_E_PARSE, a.line, "expected [register+offset]");
        RawOperand ar;
        ar.kind = RawOperand::WORD;
        ar.text = a.text;
        ar.line = a.line;
        const RegInfo& base_reg = reg_of(ar);
        if (base_reg.width == 1) raise(KS_E_PARSE, a.line, "address base %s is a predicate", a.text.c_str());
        Operand ao;
        ao.kind = KK_REG;
        ao.slot = (uint8_t)base_reg.slot;
        ao.sb = (uint8_t)base_reg.sb;
        set_src(in, 0, ao);
        // the address register's width goes into imm[0]'s unused space: 32 or 64
        in.imm[0] = (uint64_t)base_reg.width;
        in.off = a.mem_off;
        if (ld) {
          set_dst_reg(in, ops[0], td.width);
        } else {
          const RawOperand& v = ops[1];
          if (v.kind != RawOperand::WORD || !regs.count(v.text)) raise(KS_E_UNSUPPORTED, v.line, "store value must be a register");
          set_src(in, 1, value_src(v, td.width, td.is_float, false));
        }
      } else {
        raise(KS_E_UNSUPPORTED, d.line, "unsupported state space .%s", space.c_str());
      }
    } else if (base == "bra") {
      if (!(m.size() == 1 || (m.size() == 2 && m[1] == "uni"))) bad_form();
      nops(1);
      if (ops[0].kind != RawOperand::WORD) raise(KS_E_PARSE, d.line, "bra needs a label");
      in.op = KO_BRA;
      lat_class = KS_LAT_BRA;
      d.target_label = ops[0].text;
      d.is_branch = true;
    } else if (base == "bar") {
      if (!(m.size() == 2 && m[1] == "sync")) bad_form();
      nops(1);
      uint64_t v;
      if (ops[0].kind != RawOperand::NUM || !parse_u64(ops[0].text, v) || v != 0 || ops[0].neg)
        raise(KS_E_UNSUPPORTED, d.line, "only bar.sync 0 is supported");
      if (d.guarded) raise(KS_E_UNSUPPORTED, d.line, "guarded bar.sync is not supported");
      in.op = KO_BAR;
      lat_class = KS_LAT_BAR;
    } else if (base == "ret" || base == "exit") {
      if (m.size() != 1) bad_form();
      nops(0);
      in.op = KO_RET;
      lat_class = KS_LAT_RET;
      d.is_ret = true;
    } else {
      bad_form();
    }
    in.lat = lat_class;  // the class; its cycles come from the configuration when a state is allocated
    P->code.push_back(d);
  }

  void resolve_labels() {
    for (Decoded& d : P->code) {
      if (!d.is_branch) continue;
      auto it = labels.find(d.target_label);
      if (it == labels.end()) raise(KS_E_PARSE, d.line, "unknown label %s", d.target_label.c_str());
      d.in.target = (uint16_t)it->second;
    }
  }
};

// ---------------------------------------------------------------------------- reconvergence
//
// Basic blocks, a virtual exit node, and immediate post-dominators by the
// Cooper-Harvey-Kennedy iteration ("A Simple, Fast Dominance Algorithm") run on
// the reversed graph rooted at exit.  Blocks that cannot reach exit get exit.

void compute_reconvergence(ks_program* P) {
  const int n = (int)P->code.size();
  std::vector<char> leader(n + 1, 0);
  leader[0] = 1;
  for (int i = 0; i < n; ++i) {
    const Decoded& d = P->code[i];
    if (d.is_branch) {
      if (d.in.target <= n) leader[d.in.target] = 1;
      leader[i + 1] = 1;
    } else if (d.is_ret) {
      leader[i + 1] = 1;
    }
  }
  std::vector<int> block_of(n + 1, -1), first;
  for (int i = 0; i < n; ++i) {
    if (leader[i]) first.push_back(i);
    block_of[i] = (int)first.size() - 1;
  }
  const int nb = (int)first.size();
  const int EXIT = nb;
  block_of[n] = EXIT;  // falling off the end, or a label at the very end
  std::vector<std::vector<int>> succ(nb + 1), pred(nb + 1);
  for (int b = 0; b < nb; ++b) {
    int last = (b + 1 < nb ? first[b + 1] : n) - 1;
    const Decoded& d = P->code[last];
    std::vector<int> s;
    if (d.is_branch) {
      s.push_back(block_of[d.in.target]);
      if (d.guarded) s.push_back(block_of[last + 1]);
    } else if (d.is_ret) {
      s.push_back(EXIT);
      if (d.guarded) s.push_back(block_of[last + 1]);
    } else {
      s.push_back(block_of[last + 1]);
    }
    std::sort(s.begin(), s.end());
    s.erase(std::unique(s.begin(), s.end()), s.end());
    succ[b] = s;
    for (int x : s) pred[x].push_back(b);
  }
  // postorder of the reverse graph from EXIT (iterative DFS over predecessors)
  std::vector<int> order, po_num(nb + 1, -1);
  std::vector<char> seen(nb + 1, 0);
  std::vector<std::pair<int, size_t>> stack;
  stack.push_back({EXIT, 0});
  seen[EXIT] = 1;
  while (!stack.empty()) {
    auto& top = stack.back();
    if (top.second < pred[top.first].size()) {
      int p = pred[top.first][top.second++];
      if (!seen[p]) {
        seen[p] = 1;
        stack.push_back({p, 0});
      }
    } else {
      po_num[top.first] = (int)order.size();
      order.push_back(top.first);
      stack.pop_back();
    }
  }
  std::vector<int> ipdom(nb + 1, -1);
  ipdom[EXIT] = EXIT;
  auto intersect = [&](int a, int b) {
    while (a != b) {
      while (po_num[a] < po_num[b]) a = ipdom[a];
      while (po_num[b] < po_num[a]) b = ipdom[b];
    }
    return a;
  };
  bool changed = true;
  while (changed) {
    changed = false;
    for (int k = (int)order.size() - 1; k >= 0; --k) {  // reverse postorder
      int b = order[k];
      if (b == EXIT) continue;
      int nd = -1;
      for (int s : succ[b]) {
        if (ipdom[s] < 0) continue;
        nd = nd < 0 ? s : intersect(s, nd);
      }
      if (nd >= 0 && ipdom[b] != nd) {
        ipdom[b] = nd;
        changed = true;
      }
    }
  }
  P->rpc.assign(n, (uint32_t)n);
  for (int i = 0; i < n; ++i) {
    Decoded& d = P->code[i];
    if (!(d.is_branch && d.guarded)) {
      d.in.rpc = KS_RPC_EXIT;
      P->rpc[i] = 0xFFFFFFFFu;
      continue;
    }
    int b = block_of[i];
    int r = ipdom[b];
    if (r < 0 || r == EXIT) {
      d.in.rpc = KS_RPC_EXIT;
      P->rpc[i] = (uint32_t)n;
    } else {
      d.in.rpc = (uint16_t)first[r];
      P->rpc[i] = (uint32_t)first[r];
    }
  }
}

// ---------------------------------------------------------------------------- device records
//
// Lower the parsed records to the interpreter's DInst records (n + 1 of them: a
// DC_END sentinel after the last instruction; then KS_PREFETCH_PAD zero records
// that the interpreter may read ahead into).  Immediate source k goes to the
// immediate slots reg_slots + 2k (low) and + 2k + 1 (high); f32 add, sub and mul
// become one fused multiply-add with constant operands, which rounds exactly as
// the separate operation does (x + y = fma(x, 1, y), x - y = fma(x, 1, -y),
// x * y = fma(x, y, -0)), the constants read from the two slots after the
// immediates; integer add/sub and mul/mad differ only in constants.
std::vector<DInst> lower_program(const ks_program* P, const ks_config* cfg) {
  const uint32_t n = (uint32_t)P->code.size();
  const uint32_t ib = P->reg_slots;
  std::vector<DInst> out(n + 1 + KS_PREFETCH_PAD);
  auto sbo = [](uint8_t sb) -> uint32_t { return (uint32_t)(sb == KS_NO_SB ? KS_SB_ZERO : sb) * 4u; };
  for (uint32_t i = 0; i <= n; ++i) {
    DInst& d = out[i];
    memset(&d, 0, sizeof d);
    for (int k = 0; k < 4; ++k) d.sbo[k] = KS_SB_ZERO * 4u;
    d.sbod = KS_SB_DUMP * 4u;
    d.gmode = 2;
    if (i == n) {
      d.ctl = CB(DC_END) | XF_FIX;
      continue;
    }
    const KsInst& in = P->code[i].in;
    uint32_t slot[3];
    for (int k = 0; k < 3; ++k) {
      const uint32_t kind = (in.kinds >> (2 * k)) & 3u;
      if (kind == KK_IMM) {
        slot[k] = ib + 2u * k;
        d.imm[2 * k] = (uint32_t)in.imm[k];
        d.imm[2 * k + 1] = (uint32_t)(in.imm[k] >> 32);
        d.ctl |= XF_IMM;
      } else {
        slot[k] = kind == KK_REG ? in.src[k] : 0u;
      }
    }
    d.s0 = slot[0];
    d.s1 = slot[1];
    d.s2 = slot[2];
    d.dst = in.dst;
    for (int k = 0; k < 4; ++k) d.sbo[k] = sbo(in.sb[k]);
    d.sbod = in.sb_dst == KS_NO_SB ? KS_SB_DUMP * 4u : (uint32_t)in.sb_dst * 4u;
    d.lat = cfg->latency[in.lat];
    if (in.flags & KF_GUARD) {
      d.gp = in.guard;
      d.gmode = (in.flags & KF_GUARD_NEG) ? 1u : 0u;
    }
    uint32_t cls = DC_RET;
    switch (in.op) {
      case KO_ADD32: case KO_SUB32:
        cls = DC_IADD;
        d.a0 = in.op == KO_SUB32 ? 0xFFFFFFFFu : 0u;
        d.a1 = in.op == KO_SUB32 ? 1u : 0u;
        break;
      case KO_MUL32: case KO_MAD32:
        cls = DC_IMAD;
        d.a0 = in.op == KO_MAD32 ? 0xFFFFFFFFu : 0u;
        break;
      case KO_ADD64: case KO_SUB64: case KO_MUL64: case KO_MAD64:
        cls = DC_I64;
        d.a0 = in.op == KO_ADD64 ? DI_ADD : in.op == KO_SUB64 ? DI_SUB : in.op == KO_MUL64 ? DI_MUL : DI_MAD;
        break;
      case KO_MULWIDE_S: case KO_MULWIDE_U:
        cls = DC_I64;
        d.a0 = in.op == KO_MULWIDE_S ? DI_WIDE_S : DI_WIDE_U;
        break;
      case KO_FADD: case KO_FSUB:  // fma(x0, 1.0, +-x1): 1.0 from its constant slot, x1 the third operand
        cls = DC_FMA;
        d.s1 = ib + KS_IMM_SLOTS;
        d.s2 = slot[1];
        d.a2 = in.op == KO_FSUB ? 0x80000000u : 0u;
        break;
      case KO_FMUL:  // fma(x0, x1, -0.0): -0.0 from its constant slot
        cls = DC_FMA;
        d.s2 = ib + KS_IMM_SLOTS + 1u;
        d.a2 = 0;
        break;
      case KO_FFMA:  // fma(x0, x1, x2)
        cls = DC_FMA;
        d.a2 = 0;
        break;
      case KO_SETP_S32: case KO_SETP_U32: case KO_SETP_F32: case KO_SETP_S64: case KO_SETP_U64: {
        cls = DC_SETP;
        d.a0 = in.op == KO_SETP_S32 ? DS_S32 : in.op == KO_SETP_U32 ? DS_U32 : in.op == KO_SETP_F32 ? DS_F32
             : in.op == KO_SETP_S64 ? DS_S64 : DS_U64;
        static const uint32_t rel[6] = {2u, 5u, 1u, 3u, 4u, 6u};  // eq ne lt le gt ge over {lt, eq, gt}
        d.a1 = rel[in.cmp];
        break;
      }
      case KO_SELP32: case KO_SELP64:
        cls = DC_SELP;
        d.a0 = in.op == KO_SELP64 ? 1u : 0u;
        d.s2 = in.src[2];  // predicate index
        break;
      case KO_MOV32: case KO_MOV64:
        if ((in.kinds & 3u) == KK_SPECIAL) {
          cls = DC_MOVSP;
          d.a0 = in.src[0];
        } else {
          cls = DC_MOV;
          d.a0 = in.op == KO_MOV64 ? 1u : 0u;
        }
        break;
      case KO_LDP32: case KO_LDP64:
        cls = DC_LDP;
        d.a0 = in.aux;
        d.a1 = in.op == KO_LDP64 ? 1u : 0u;
        break;
      case KO_LDG32: case KO_LDG64: case KO_STG32: case KO_STG64:
      case KO_LDS32: case KO_LDS64: case KO_STS32: case KO_STS64: {
        const bool g = in.op <= KO_STG64;
        cls = g ? DC_MEMG : DC_MEMS;
        const bool ld = in.op == KO_LDG32 || in.op == KO_LDG64 || in.op == KO_LDS32 || in.op == KO_LDS64;
        const bool w64 = in.op == KO_LDG64 || in.op == KO_STG64 || in.op == KO_LDS64 || in.op == KO_STS64;
        if (g && !w64 && in.imm[0] == 64) cls = ld ? DC_LDG : DC_STG;  // the common form has its own class
        d.ctl |= (ld ? XF_LOAD : 0u) | (w64 ? XF_W64 : 0u) | (in.imm[0] == 64 ? XF_A64 : 0u);
        d.s0 = in.src[0];
        d.s1 = ld ? 0u : in.src[1];
        d.a0 = (uint32_t)(uint64_t)in.off;
        d.a1 = (uint32_t)((uint64_t)in.off >> 32);
        break;
      }
      case KO_BRA:
        cls = DC_BRA;
        d.a0 = in.target;
        d.a1 = in.rpc == KS_RPC_EXIT ? 0xFFFFFFFFu : in.rpc;
        break;
      case KO_BAR:
        cls = DC_BAR;
        break;
      default:
        cls = DC_RET;
        break;
    }
    d.ctl |= CB(cls);
  }
  for (uint32_t i = 0; i < n; ++i) {
    const KsInst& in = P->code[i].in;
    if (in.op == KO_BRA && in.rpc != KS_RPC_EXIT) out[in.rpc].ctl |= XF_FIX;
  }
  // each record also carries the next one's scoreboard offsets (a straight run reads
  // them with this record, so the next issue cycle does not wait for the next record)
  for (uint32_t i = 0; i < n; ++i)
    for (int k = 0; k < 4; ++k) out[i].nsbo[k] = out[i + 1].sbo[k];
  // straight runs, from the end: the run of a non-control instruction is itself and
  // the instructions after it that may follow it without rescheduling (neither a
  // control instruction, nor a reconvergence point, nor the end sentinel)
  uint32_t next = 0;  // run length of instruction i + 1, 0 if it cannot continue a run
  for (uint32_t i = n; i-- > 0;) {
    const uint32_t run = (out[i].ctl & CB_CTRL) ? 1u : (next + 1u > RUN_MAX ? RUN_MAX : next + 1u);
    out[i].ctl |= run << RUN_SHIFT;
    next = (out[i].ctl & (CB_CTRL | XF_FIX)) ? 0u : run;
  }
  return out;
}

template <class F>
ks_status guarded(F&& f) {
  try {
    g_last_error.clear();
    return f();
  } catch (const KsFail& e) {
    return e.code;
  } catch (const std::bad_alloc&) {
    g_last_error = "host allocation failed";
    return KS_E_NOMEM;
  } catch (...) {
    g_last_error = "internal error";
    return KS_E_INVALID_ARG;
  }
}

bool hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return false;
}

}  // namespace

struct ks_state {
  const ks_program* prog;
  ks_config cfg;
  int device;
  DInst* d_prog;
  void* d_gmem;
  void* d_counters;
  void* d_trace;
  void* d_cache;              // the cache model's per-warp state (NULL without it)
  uint32_t* d_status;
  uint64_t last_warps = 0;    // warps of the last run (0 = no run yet)
  uint64_t slot_bytes;
  uint64_t max_warps;
  bool in_scratch = false;    // program and status word live in the library's static scratch
  uint64_t generation = 0;    // its binding generation on `device` (in_scratch only)
};

// ---------------------------------------------------------------------------- ABI

extern "C" {

const char* ks_last_error(void) { return g_last_error.c_str(); }

ks_status ks_load_program(const char* ptx, size_t len, const char* entry, ks_program** out) {
  return guarded([&]() -> ks_status {
    if (!ptx || !out) raise(KS_E_INVALID_ARG, 0, "NULL argument");
    *out = nullptr;
    std::vector<Tok> toks = lex(ptx, len);
    Front f(toks);
    ks_program* p = f.run(entry);
    try {
      compute_reconvergence(p);
    } catch (...) {
      delete p;
      throw;
    }
    *out = p;
    return KS_OK;
  });
}

void ks_program_free(ks_program* p) { delete p; }

ks_status ks_program_info(const ks_program* p, ks_program_desc* out) {
  return guarded([&]() -> ks_status {
    if (!p || !out) raise(KS_E_INVALID_ARG, 0, "NULL argument");
    out->n_instrs = (uint32_t)p->code.size();
    out->n_params = (uint32_t)p->params.size();
    out->param_bytes = p->param_bytes;
    out->shared_bytes = p->shared_bytes;
    out->reg_slots = p->reg_slots;
    out->n_preds = p->n_preds;
    return KS_OK;
  });
}

ks_status ks_param_info(const ks_program* p, uint32_t index, uint32_t* offset, uint32_t* size, const char** name) {
  return guarded([&]() -> ks_status {
    if (!p) raise(KS_E_INVALID_ARG, 0, "NULL program");
    if (index >= p->params.size()) raise(KS_E_INVALID_ARG, 0, "parameter index %u out of range", index);
    if (offset) *offset = p->params[index].offset;
    if (size) *size = p->params[index].size;
    if (name) *name = p->params[index].name.c_str();
    return KS_OK;
  });
}

ks_status ks_param_offset(const ks_program* p, const char* name, uint32_t* offset, uint32_t* size) {
  return guarded([&]() -> ks_status {
    if (!p || !name) raise(KS_E_INVALID_ARG, 0, "NULL argument");
    for (const auto& prm : p->params) {
      if (prm.name == name) {
        if (offset) *offset = prm.offset;
        if (size) *size = prm.size;
        return KS_OK;
      }
    }
    raise(KS_E_INVALID_ARG, 0, "no parameter named '%s'", name);
  });
}

ks_status ks_instr_info(const ks_program* p, uint32_t pc, ks_instr_desc* out) {
  return guarded([&]() -> ks_status {
    if (!p || !out) raise(KS_E_INVALID_ARG, 0, "NULL argument");
    if (pc >= p->code.size()) raise(KS_E_INVALID_ARG, 0, "pc %u outside the program (%zu instructions)", pc, p->code.size());
    const Decoded& d = p->code[pc];
    const KsInst& in = d.in;
    memset(out, 0, sizeof *out);
    out->line = (uint32_t)d.line;
    out->lat_class = in.lat;
    switch (in.op) {
      case KO_LDG32: case KO_LDG64: out->kind = KS_EV_LD_GLOBAL; break;
      case KO_STG32: case KO_STG64: out->kind = KS_EV_ST_GLOBAL; break;
      case KO_LDS32: case KO_LDS64: out->kind = KS_EV_LD_SHARED; break;
      case KO_STS32: case KO_STS64: out->kind = KS_EV_ST_SHARED; break;
      case KO_BRA: out->kind = KS_EV_BRANCH; break;
      case KO_BAR: out->kind = KS_EV_BARRIER; break;
      case KO_RET: out->kind = KS_EV_RET; break;
      default: out->kind = KS_EV_OTHER; break;
    }
    if (out->kind >= KS_EV_LD_GLOBAL && out->kind <= KS_EV_ST_SHARED)
      out->access_bytes = (in.op == KO_LDG64 || in.op == KO_STG64 || in.op == KO_LDS64 || in.op == KO_STS64) ? 8u : 4u;
    return KS_OK;
  });
}

ks_status ks_ipdom_table(const ks_program* p, uint32_t* out, uint32_t n) {
  return guarded([&]() -> ks_status {
    if (!p || (!out && n)) raise(KS_E_INVALID_ARG, 0, "NULL argument");
    for (uint32_t i = 0; i < n && i < p->rpc.size(); ++i) out[i] = p->rpc[i];
    return KS_OK;
  });
}

ks_status ks_default_config(ks_config* cfg) {
  return guarded([&]() -> ks_status {
    if (!cfg) raise(KS_E_INVALID_ARG, 0, "NULL config");
    memset(cfg, 0, sizeof *cfg);
    cfg->max_grid = {1, 1, 1};
    cfg->max_block = {1, 1, 1};
    cfg->max_warp_instrs = 0xFFFFFFFFu;
    // sm_80 latency model of the KernelScope latency page; classes it does not list
    // take the integer/control value of 4 (ld.param as the constant-bank ld.const).
    uint16_t* L = cfg->latency;
    L[KS_LAT_INT32] = 4;
    L[KS_LAT_INT64] = 4;
    L[KS_LAT_FP32] = 4;
    L[KS_LAT_SETP] = 4;
    L[KS_LAT_SELP] = 4;
    L[KS_LAT_MOV] = 4;
    L[KS_LAT_LD_PARAM] = 4;
    L[KS_LAT_LD_GLOBAL] = 200;
    L[KS_LAT_LD_SHARED] = 23;
    L[KS_LAT_ST_GLOBAL] = 200;
    L[KS_LAT_ST_SHARED] = 23;
    L[KS_LAT_BRA] = 4;
    L[KS_LAT_BAR] = 20;
    // cache model: the cache latencies of the KernelScope memory-analysis part
    L[KS_LAT_L1_HIT] = 28;
    L[KS_LAT_L2_HIT] = 150;
    L[KS_LAT_DRAM] = 400;
    L[KS_LAT_RET] = 4;
    return KS_OK;
  });
}

static uint64_t dim_count(const ks_dim3& d) { return (uint64_t)d.x * d.y * d.z; }

ks_status ks_query_layout(const ks_program* p, const ks_config* cfg, ks_layout* out) {
  return guarded([&]() -> ks_status {
    if (!p || !cfg || !out) raise(KS_E_INVALID_ARG, 0, "NULL argument");
    uint64_t tpb = dim_count(cfg->max_block);
    uint64_t nb = dim_count(cfg->max_grid);
    if (tpb == 0 || nb == 0) raise(KS_E_INVALID_ARG, 0, "zero grid or block dimension");
    if (tpb > KS_MAX_BLOCK_THREADS) raise(KS_E_INVALID_ARG, 0, "more than %d threads per block", KS_MAX_BLOCK_THREADS);
    memset(out, 0, sizeof *out);
    out->warps_per_block = (uint32_t)((tpb + 31) / 32);
    out->n_warps = nb * out->warps_per_block;
    out->counters_bytes = out->n_warps * 80;
    if (cfg->trace_format != KS_TRACE_BASIC && cfg->trace_format != KS_TRACE_EXTENDED)
      raise(KS_E_INVALID_ARG, 0, "unknown trace format %u", cfg->trace_format);
    if (cfg->trace_format == KS_TRACE_EXTENDED) {
      const uint32_t lim = ks_choose_variant(p->reg_slots, (uint32_t)tpb) == 64 ? KS_EXT64_MAX_BLOCK_THREADS : KS_EXT_MAX_BLOCK_THREADS;
      if (tpb > lim)
        raise(KS_E_UNSUPPORTED, 0, "extended trace records of programs with %u register slots support blocks of up to %u threads",
              p->reg_slots, lim);
    }
    if (cfg->cache_model != KS_CACHE_NONE && cfg->cache_model != KS_CACHE_WARP)
      raise(KS_E_INVALID_ARG, 0, "unknown cache model %u", cfg->cache_model);
    if (cfg->cache_model == KS_CACHE_WARP) {
      if (cfg->trace_format != KS_TRACE_BASIC) raise(KS_E_UNSUPPORTED, 0, "the cache model runs with basic trace records");
      // valid addresses give line numbers below 2^31: tags (line + 1) fit 32 bits
      if (cfg->gmem_bytes > (1ull << 38)) raise(KS_E_UNSUPPORTED, 0, "the cache model covers at most 2^38 bytes");
    }
    out->slot_bytes = 16 + (cfg->trace_format == KS_TRACE_EXTENDED ? 16 : 8) * (uint64_t)cfg->trace_cap;
    out->trace_bytes = out->n_warps * out->slot_bytes;
    out->cache_bytes = cfg->cache_model == KS_CACHE_WARP ? out->n_warps * (uint64_t)KS_CACHE_WARP_BYTES : 0;
    return KS_OK;
  });
}

ks_status ks_alloc_state(const ks_program* p, const ks_config* cfg, void* d_gmem, void* d_counters, void* d_trace,
                         void* d_cache, ks_state** out) {
  return guarded([&]() -> ks_status {
    if (!p || !cfg || !out) raise(KS_E_INVALID_ARG, 0, "NULL argument");
    *out = nullptr;
    if (!d_gmem || !d_counters || !d_trace) raise(KS_E_INVALID_ARG, 0, "NULL device buffer");
    if (cfg->cache_model == KS_CACHE_WARP && !d_cache) raise(KS_E_INVALID_ARG, 0, "NULL cache buffer");
    if (cfg->cache_model == KS_CACHE_WARP && ((uintptr_t)d_cache & 15u))
      raise(KS_E_INVALID_ARG, 0, "cache buffer not 16-byte aligned");
    if (p->reg_slots > KS_MAX_REG_SLOTS) raise(KS_E_UNSUPPORTED, 0, "program needs %u register slots (limit %d)", p->reg_slots, KS_MAX_REG_SLOTS);
    if (p->n_preds > KS_MAX_PREDS) raise(KS_E_UNSUPPORTED, 0, "program needs %u predicates (limit %d)", p->n_preds, KS_MAX_PREDS);
    if (p->code.empty()) raise(KS_E_INVALID_ARG, 0, "empty program");
    ks_layout lay;
    ks_status s = ks_query_layout(p, cfg, &lay);
    if (s != KS_OK) return s;
    int dev = -1;
    if (!hip_ok(hipGetDevice(&dev), "hipGetDevice")) return KS_E_HIP;
    hipDeviceProp_t prop;
    if (!hip_ok(hipGetDeviceProperties(&prop, dev), "hipGetDeviceProperties")) return KS_E_HIP;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) raise(KS_E_HIP, 0, "device %d is %s, not gfx950", dev, prop.gcnArchName);
    const std::vector<DInst> table = lower_program(p, cfg);
    DInst* d_prog = nullptr;
    uint32_t* d_status = nullptr;
    if (!hip_ok(hipMalloc((void**)&d_prog, table.size() * sizeof(DInst)), "hipMalloc(program)")) return KS_E_NOMEM;
    if (!hip_ok(hipMalloc((void**)&d_status, 256), "hipMalloc(status)")) {
      (void)hipFree(d_prog);
      return KS_E_NOMEM;
    }
    if (!hip_ok(hipMemcpy(d_prog, table.data(), table.size() * sizeof(DInst), hipMemcpyHostToDevice), "hipMemcpy(program)")) {
      (void)hipFree(d_prog);
      (void)hipFree(d_status);
      return KS_E_HIP;
    }
    ks_state* st = new ks_state();
    st->prog = p;
    st->cfg = *cfg;
    st->device = dev;
    st->d_prog = d_prog;
    st->d_gmem = d_gmem;
    st->d_counters = d_counters;
    st->d_trace = d_trace;
    st->d_cache = cfg->cache_model == KS_CACHE_WARP ? d_cache : nullptr;
    st->d_status = d_status;
    st->slot_bytes = lay.slot_bytes;
    st->max_warps = lay.n_warps;
    *out = st;
    return KS_OK;
  });
}

ks_status ks_alloc_state_static(const ks_program* p, const ks_config* cfg, void* d_gmem, void* d_counters,
                                void* d_trace, void* d_cache, ks_state** out) {
  return guarded([&]() -> ks_status {
    if (!p || !cfg || !out) raise(KS_E_INVALID_ARG, 0, "NULL argument");
    *out = nullptr;
    if (!d_gmem || !d_counters || !d_trace) raise(KS_E_INVALID_ARG, 0, "NULL device buffer");
    if (cfg->cache_model == KS_CACHE_WARP && !d_cache) raise(KS_E_INVALID_ARG, 0, "NULL cache buffer");
    if (cfg->cache_model == KS_CACHE_WARP && ((uintptr_t)d_cache & 15u))
      raise(KS_E_INVALID_ARG, 0, "cache buffer not 16-byte aligned");
    if (p->reg_slots > KS_MAX_REG_SLOTS) raise(KS_E_UNSUPPORTED, 0, "program needs %u register slots (limit %d)", p->reg_slots, KS_MAX_REG_SLOTS);
    if (p->n_preds > KS_MAX_PREDS) raise(KS_E_UNSUPPORTED, 0, "program needs %u predicates (limit %d)", p->n_preds, KS_MAX_PREDS);
    if (p->code.empty()) raise(KS_E_INVALID_ARG, 0, "empty program");
    if (p->code.size() > KS_STATIC_MAX_INSTRS)
      raise(KS_E_UNSUPPORTED, 0, "program of %zu instructions exceeds the static scratch (at most %d instructions)",
            p->code.size(), KS_STATIC_MAX_INSTRS);
    ks_layout lay;
    ks_status s = ks_query_layout(p, cfg, &lay);
    if (s != KS_OK) return s;
    int dev = -1;
    if (!hip_ok(hipGetDevice(&dev), "hipGetDevice")) return KS_E_HIP;
    hipDeviceProp_t prop;
    if (!hip_ok(hipGetDeviceProperties(&prop, dev), "hipGetDeviceProperties")) return KS_E_HIP;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) raise(KS_E_HIP, 0, "device %d is %s, not gfx950", dev, prop.gcnArchName);
    const std::vector<DInst> table = lower_program(p, cfg);
    DInst* d_prog = nullptr;
    uint32_t* d_status = nullptr;
    uint64_t gen = 0;
    if (!hip_ok(ks_static_scratch(dev, &d_prog, &d_status, &gen), "static scratch address")) return KS_E_HIP;
    if (!hip_ok(hipMemcpy(d_prog, table.data(), table.size() * sizeof(DInst), hipMemcpyHostToDevice), "hipMemcpy(program)"))
      return KS_E_HIP;
    ks_state* st = new ks_state();
    st->prog = p;
    st->cfg = *cfg;
    st->device = dev;
    st->d_prog = d_prog;
    st->d_gmem = d_gmem;
    st->d_counters = d_counters;
    st->d_trace = d_trace;
    st->d_cache = cfg->cache_model == KS_CACHE_WARP ? d_cache : nullptr;
    st->d_status = d_status;
    st->slot_bytes = lay.slot_bytes;
    st->max_warps = lay.n_warps;
    st->in_scratch = true;
    st->generation = gen;
    *out = st;
    return KS_OK;
  });
}

void ks_state_free(ks_state* st) {
  if (!st) return;
  if (!st->in_scratch) {
    (void)hipFree(st->d_prog);
    (void)hipFree(st->d_status);
  }
  delete st;
}

ks_status ks_run(ks_state* st, ks_dim3 grid, ks_dim3 block, const void* params, size_t params_len, void* stream) {
  return guarded([&]() -> ks_status {
    if (!st) raise(KS_E_INVALID_ARG, 0, "NULL state");
    if (st->in_scratch && ks_static_generation(st->device) != st->generation)
      raise(KS_E_STATE, 0, "another static state was bound on device %d since this one: its program is gone", st->device);
    const ks_program* p = st->prog;
    if (!grid.x || !grid.y || !grid.z || !block.x || !block.y || !block.z) raise(KS_E_INVALID_ARG, 0, "zero grid or block dimension");
    uint64_t tpb = dim_count(block), nb = dim_count(grid);
    if (tpb > dim_count(st->cfg.max_block) || nb > dim_count(st->cfg.max_grid))
      raise(KS_E_INVALID_ARG, 0, "grid/block larger than the allocation");
    if (tpb > KS_MAX_BLOCK_THREADS) raise(KS_E_INVALID_ARG, 0, "more than %d threads per block", KS_MAX_BLOCK_THREADS);
    if (nb > 0x7FFFFFFFull) raise(KS_E_INVALID_ARG, 0, "too many blocks");
    if (st->cfg.trace_format == KS_TRACE_EXTENDED) {
      const uint32_t lim = ks_choose_variant(p->reg_slots, (uint32_t)tpb) == 64 ? KS_EXT64_MAX_BLOCK_THREADS : KS_EXT_MAX_BLOCK_THREADS;
      if (tpb > lim)
        raise(KS_E_UNSUPPORTED, 0, "extended trace records of programs with %u register slots support blocks of up to %u threads",
              p->reg_slots, lim);
    }
    if (params_len < p->param_bytes || (p->param_bytes && !params)) raise(KS_E_INVALID_ARG, 0, "parameter block shorter than %u bytes", p->param_bytes);
    KsArgs a;
    memset(&a, 0, sizeof a);
    a.prog = st->d_prog;
    a.gmem = (uint8_t*)st->d_gmem;
    a.counters = (uint8_t*)st->d_counters;
    a.trace = (uint8_t*)st->d_trace;
    a.gmem_bytes = st->cfg.gmem_bytes;
    a.slot_bytes = st->slot_bytes;
    a.n_instrs = (uint32_t)p->code.size();
    a.trace_cap = st->cfg.trace_cap;
    a.max_warp_instrs = st->cfg.max_warp_instrs;
    a.shared_bytes = p->shared_bytes;
    a.grid[0] = grid.x;
    a.grid[1] = grid.y;
    a.grid[2] = grid.z;
    a.block[0] = block.x;
    a.block[1] = block.y;
    a.block[2] = block.z;
    a.threads_per_block = (uint32_t)tpb;
    a.warps_per_block = (uint32_t)((tpb + 31) / 32);
    a.lat_bar = st->cfg.latency[KS_LAT_BAR];
    {
      // each issue of a run is at most (the largest latency + 1) after the previous one
      uint64_t step = 1;
      for (int k = 0; k < KS_NLAT; ++k) step = std::max<uint64_t>(step, (uint64_t)st->cfg.latency[k] + 1);
      const uint64_t limit = 0x7FFFFFFFull, span = (uint64_t)RUN_MAX * step;
      a.cyc_safe = span < limit ? (uint32_t)(limit - span) : 0u;
    }
    a.rf_slots = p->reg_slots + KS_IMM_SLOTS + KS_CONST_SLOTS;
    a.ext = st->cfg.trace_format == KS_TRACE_EXTENDED ? 1u : 0u;
    a.cache = (uint8_t*)st->d_cache;
    a.cache_on = st->d_cache ? 1u : 0u;
    a.lat_l1 = st->cfg.latency[KS_LAT_L1_HIT];
    a.lat_l2 = st->cfg.latency[KS_LAT_L2_HIT];
    a.lat_dram = st->cfg.latency[KS_LAT_DRAM];
    // %tid.y and %tid.z divide the linear thread index (< 1024) by block sizes (<= 1024):
    // (t * ceil(2^22 / d)) >> 22 == t / d over that range, with no 32-bit overflow
    auto recip22 = [](uint64_t d) { return (uint32_t)(((1ull << 22) + d - 1) / d); };
    a.div_bx = recip22(block.x);
    a.div_by = recip22(block.y);
    a.div_bxy = recip22((uint64_t)block.x * block.y);
    if (p->param_bytes) memcpy(a.params, params, p->param_bytes);
    uint64_t warps = nb * a.warps_per_block;
    if (warps > st->max_warps) raise(KS_E_INVALID_ARG, 0, "run needs more warps than the allocation");
    {
      const int variant = ks_choose_variant(p->reg_slots, a.threads_per_block);
      if (variant == 0) raise(KS_E_UNSUPPORTED, 0, "program needs %u register slots", p->reg_slots);
      const uint32_t wg = 64u * ((a.warps_per_block + 1u) / 2u);
      if (wg > ks_max_block_threads(variant, a.ext != 0))
        raise(KS_E_UNSUPPORTED, 0, "extended trace records with %u register slots support blocks of up to %u threads",
              p->reg_slots, ks_max_block_threads(variant, true));
      const size_t need = ks_lds_bytes(wg, p->shared_bytes, a.ext != 0);
      if (need + 64 > ks_lds_limit())
        raise(KS_E_UNSUPPORTED, 0, "block of %u threads needs %zu bytes of LDS (limit %zu)", a.threads_per_block, need,
              ks_lds_limit() - 64);
    }
    if (a.cache_on) {
      // the caches of this run's warps start empty
      if (!hip_ok(ks_launch_clear(st->d_cache, warps * (uint64_t)KS_CACHE_WARP_BYTES, (hipStream_t)stream),
                  "clearing the cache state"))
        return KS_E_HIP;
    }
    // Extended records run as launches of at most KS_EXT_MAX_BLOCKS blocks, one after
    // another on the stream; a basic or cache-model run is one launch.
    const uint64_t chunk = a.ext ? (uint64_t)KS_EXT_MAX_BLOCKS : nb;
    for (uint64_t b0 = 0; b0 < nb; b0 += chunk) {
      a.block_base = (uint32_t)b0;
      hipError_t e = ks_launch_interp(a, (uint32_t)std::min<uint64_t>(chunk, nb - b0), p->reg_slots, (hipStream_t)stream);
      if (!hip_ok(e, "kernel launch")) return KS_E_HIP;
    }
    st->last_warps = warps;
    return KS_OK;
  });
}

ks_status ks_interp_kernel(const ks_program* prog, ks_dim3 block, const char** name) {
  return guarded([&]() -> ks_status {
    if (!prog || !name) raise(KS_E_INVALID_ARG, 0, "NULL argument");
    const uint64_t tpb = dim_count(block);
    if (!tpb || tpb > KS_MAX_BLOCK_THREADS) raise(KS_E_INVALID_ARG, 0, "block of %llu threads", (unsigned long long)tpb);
    const int variant = ks_choose_variant(prog->reg_slots, (uint32_t)tpb);
    if (variant == 0) raise(KS_E_UNSUPPORTED, 0, "program needs %u register slots", prog->reg_slots);
    *name = variant == 32 ? "ks_interp_v32" : "ks_interp_v64";
    return KS_OK;
  });
}

ks_status ks_read_outputs(ks_state* st, uint64_t sim_addr, void* host, size_t n, void* stream) {
  return guarded([&]() -> ks_status {
    if (!st || (!host && n)) raise(KS_E_INVALID_ARG, 0, "NULL argument");
    if (sim_addr > st->cfg.gmem_bytes || n > st->cfg.gmem_bytes - sim_addr) raise(KS_E_INVALID_ARG, 0, "range outside simulated memory");
    if (!n) return KS_OK;
    hipStream_t s = (hipStream_t)stream;
    if (!hip_ok(hipMemcpyAsync(host, (uint8_t*)st->d_gmem + sim_addr, n, hipMemcpyDeviceToHost, s), "hipMemcpyAsync")) return KS_E_HIP;
    if (!hip_ok(hipStreamSynchronize(s), "hipStreamSynchronize")) return KS_E_HIP;
    return KS_OK;
  });
}

static ks_status read_per_warp(ks_state* st, const void* base, uint64_t stride, uint64_t first, uint64_t count, void* host,
                               size_t n, void* stream) {
  if (!st->last_warps) raise(KS_E_STATE, 0, "no run yet");
  if (first > st->last_warps || count > st->last_warps - first) raise(KS_E_INVALID_ARG, 0, "warp range outside the last run");
  if (n < count * stride) raise(KS_E_INVALID_ARG, 0, "host buffer too small");
  if (!count) return KS_OK;
  hipStream_t s = (hipStream_t)stream;
  if (!hip_ok(hipMemcpyAsync(host, (const uint8_t*)base + first * stride, count * stride, hipMemcpyDeviceToHost, s), "hipMemcpyAsync"))
    return KS_E_HIP;
  if (!hip_ok(hipStreamSynchronize(s), "hipStreamSynchronize")) return KS_E_HIP;
  return KS_OK;
}

ks_status ks_read_counters(ks_state* st, uint64_t first_warp, uint64_t n_warps, void* host, size_t n, void* stream) {
  return guarded([&]() -> ks_status {
    if (!st || (!host && n)) raise(KS_E_INVALID_ARG, 0, "NULL argument");
    return read_per_warp(st, st->d_counters, 80, first_warp, n_warps, host, n, stream);
  });
}

ks_status ks_read_trace(ks_state* st, uint64_t first_warp, uint64_t n_warps, void* host, size_t n, void* stream) {
  return guarded([&]() -> ks_status {
    if (!st || (!host && n)) raise(KS_E_INVALID_ARG, 0, "NULL argument");
    return read_per_warp(st, st->d_trace, st->slot_bytes, first_warp, n_warps, host, n, stream);
  });
}

// ---------------------------------------------------------------------------- trace-event export

namespace {

// Buffered text output with integer formatting of its own (the export writes some
// hundred million numbers for a large slice).
struct JsonOut {
  FILE* f;
  std::string buf;
  explicit JsonOut(FILE* fp) : f(fp) { buf.reserve(1u << 23); }
  void put(const char* s) { buf.append(s); }
  void put(const char* s, size_t n) { buf.append(s, n); }
  void num(uint64_t v) {
    char t[24];
    int n = 0;
    do {
      t[n++] = (char)('0' + v % 10u);
      v /= 10u;
    } while (v);
    while (n) buf.push_back(t[--n]);
  }
  void hex8(uint32_t v) {
    static const char* d = "0123456789abcdef";
    for (int k = 7; k >= 0; --k) buf.push_back(d[(v >> (4 * k)) & 15u]);
  }
  bool flush(bool force) {
    if (!force && buf.size() < (1u << 22)) return true;
    const bool ok = fwrite(buf.data(), 1, buf.size(), f) == buf.size();
    buf.clear();
    return ok;
  }
};

const char* const kEvNames[9] = {"other", "ld.global", "st.global", "ld.shared", "st.shared", "branch", "diverge", "barrier", "ret"};

}  // namespace

ks_status ks_write_trace_events(const void* trace, uint64_t n_warps, uint64_t slot_bytes, uint32_t trace_format,
                                uint64_t first_warp, uint32_t warps_per_block, uint32_t n_pcs,
                                const char* const* pc_names, const char* const* pc_args, const char* path,
                                uint64_t* n_events) {
  return guarded([&]() -> ks_status {
    if ((!trace && n_warps) || !path || (n_pcs && (!pc_names || !pc_args)) || !warps_per_block)
      raise(KS_E_INVALID_ARG, 0, "NULL argument or zero warps per block");
    if (trace_format != KS_TRACE_BASIC && trace_format != KS_TRACE_EXTENDED)
      raise(KS_E_INVALID_ARG, 0, "unknown trace format %u", trace_format);
    for (uint32_t k = 0; k < n_pcs; ++k)
      if (!pc_names[k] || !pc_args[k]) raise(KS_E_INVALID_ARG, 0, "NULL name or args fragment of pc %u", k);
    const uint64_t rec = trace_format == KS_TRACE_EXTENDED ? 16u : 8u;
    if (slot_bytes < 16u || (slot_bytes - 16u) % rec) raise(KS_E_INVALID_ARG, 0, "slot of %llu bytes", (unsigned long long)slot_bytes);
    const uint64_t cap = (slot_bytes - 16u) / rec;
    FILE* f = fopen(path, "wb");
    if (!f) raise(KS_E_INVALID_ARG, 0, "cannot open %s", path);
    JsonOut o(f);
    uint64_t events = 0;
    bool first = true, ok = true;
    o.put("{\"traceEvents\":[");
    const uint8_t* base = static_cast<const uint8_t*>(trace);
    for (uint64_t wl = 0; wl < n_warps && ok; ++wl) {
      const uint8_t* slot = base + wl * slot_bytes;
      uint32_t written;
      memcpy(&written, slot, 4);
      if (written > cap) {
        fclose(f);
        raise(KS_E_INVALID_ARG, 0, "warp %llu: %u records in a slot of %llu", (unsigned long long)(first_warp + wl), written,
              (unsigned long long)cap);
      }
      if (!written) continue;
      const uint64_t w = first_warp + wl;
      const uint64_t b = w / warps_per_block, wib = w % warps_per_block;
      if (wib == 0) {
        o.put(first ? "" : ",");
        o.put("{\"ph\":\"M\",\"name\":\"process_name\",\"pid\":");
        o.num(b);
        o.put(",\"tid\":0,\"args\":{\"name\":\"block ");
        o.num(b);
        o.put("\"}}");
        first = false;
      }
      o.put(first ? "" : ",");
      o.put("{\"ph\":\"M\",\"name\":\"thread_name\",\"pid\":");
      o.num(b);
      o.put(",\"tid\":");
      o.num(wib);
      o.put(",\"args\":{\"name\":\"warp ");
      o.num(wib);
      o.put("\"}}");
      first = false;
      const uint8_t* r = slot + 16;
      for (uint32_t k = 0; k < written; ++k, r += rec) {
        uint32_t cyc, pc, kind = 0, active = 0, pay = 0, next = 0;
        memcpy(&cyc, r, 4);
        if (trace_format == KS_TRACE_EXTENDED) {
          uint32_t w1;
          memcpy(&w1, r + 4, 4);
          pc = w1 & 0xFFFFu;
          kind = (w1 >> 16) & 0xFFu;
          memcpy(&active, r + 8, 4);
          memcpy(&pay, r + 12, 4);
        } else {
          memcpy(&pc, r + 4, 4);
        }
        if (pc >= n_pcs || kind > KS_EV_RET) {
          fclose(f);
          raise(KS_E_INVALID_ARG, 0, "warp %llu record %u: pc %u / kind %u outside the program", (unsigned long long)w, k, pc, kind);
        }
        if (k + 1 < written) memcpy(&next, r + rec, 4);
        const uint64_t dur = k + 1 < written ? (uint64_t)next - cyc : 1u;
        o.put(",{\"ph\":\"X\",\"name\":");
        o.put(pc_names[pc]);
        o.put(",\"cat\":\"");
        o.put(trace_format == KS_TRACE_EXTENDED ? kEvNames[kind] : "issue");
        o.put("\",\"pid\":");
        o.num(b);
        o.put(",\"tid\":");
        o.num(wib);
        o.put(",\"ts\":");
        o.num(cyc);
        o.put(",\"dur\":");
        o.num(dur);
        o.put(",\"args\":{");
        o.put(pc_args[pc]);
        if (trace_format == KS_TRACE_EXTENDED) {
          o.put(",\"active\":\"0x");
          o.hex8(active);
          o.put("\"");
          if (kind == KS_EV_LD_GLOBAL || kind == KS_EV_ST_GLOBAL) {
            o.put(",\"sectors\":"); o.num(pay & 0xFFu);
            o.put(",\"lines\":"); o.num((pay >> 8) & 0xFFu);
            o.put(",\"lanes\":"); o.num((pay >> 16) & 0xFFu);
            o.put(",\"faults\":"); o.num(pay >> 24);
          } else if (kind == KS_EV_LD_SHARED || kind == KS_EV_ST_SHARED) {
            o.put(",\"degree\":"); o.num(pay & 0xFFu);
            o.put(",\"lanes\":"); o.num((pay >> 16) & 0xFFu);
            o.put(",\"faults\":"); o.num(pay >> 24);
          } else if (kind == KS_EV_BRANCH || kind == KS_EV_DIVERGE) {
            o.put(",\"taken\":"); o.num(pay);
          } else if (kind != KS_EV_BARRIER) {
            o.put(",\"guard_lanes\":"); o.num(pay);
          }
        }
        o.put("}}");
        ++events;
        ok = o.flush(false);
      }
    }
    o.put("],\"displayTimeUnit\":\"ns\",\"otherData\":{\"time_unit\":\"simulated cycle\","
          "\"source\":\"libkscope per-warp trace slots\"}}");
    ok = ok && o.flush(true);
    ok = (fclose(f) == 0) && ok;
    if (!ok) raise(KS_E_INVALID_ARG, 0, "writing %s failed", path);
    if (n_events) *n_events = events;
    return KS_OK;
  });
}

ks_status ks_run_status(ks_state* st, uint32_t* or_bits, void* stream) {
  return guarded([&]() -> ks_status {
    if (!st || !or_bits) raise(KS_E_INVALID_ARG, 0, "NULL argument");
    if (!st->last_warps) raise(KS_E_STATE, 0, "no run yet");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = ks_launch_status_or(st->d_counters, st->last_warps, st->d_status, s);
    if (!hip_ok(e, "status reduction")) return KS_E_HIP;
    if (!hip_ok(hipMemcpyAsync(or_bits, st->d_status, 4, hipMemcpyDeviceToHost, s), "hipMemcpyAsync")) return KS_E_HIP;
    if (!hip_ok(hipStreamSynchronize(s), "hipStreamSynchronize")) return KS_E_HIP;
    return KS_OK;
  });
}

}  // extern "C"
