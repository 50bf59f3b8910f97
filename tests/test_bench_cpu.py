"""Host logic of bench.py: which committed counter summaries still describe the kernel code."""

import bench


def test_code_text_drops_comments_and_layout_only():
    src = 'int a = 1;  // one\n/* two\n   lines */ const char* s = "a//b /*c*/";\nchar q = \'/\';   int b = 2; // end'
    assert bench._code_text(src) == 'int a = 1; const char* s = "a//b /*c*/"; char q = \'/\'; int b = 2;'
    # a comment edit leaves the code text unchanged, a code edit does not
    assert bench._code_text(src.replace("// one", "// first")) == bench._code_text(src)
    assert bench._code_text(src.replace("int b = 2", "int b = 3")) != bench._code_text(src)
    # escaped quotes inside a literal do not end it
    assert bench._code_text('f("x\\" // y"); // z') == 'f("x\\" // y");'

